// Fused attention backward for gfx950: dQ, dK, dV of O = softmax(scale Q K^T +
// causal mask) V for an upstream gradient dO.
//
// What it computes ("Skill: Write a Triton Attention Kernel", Do not use this
// when: the backward recomputes the attention weights from the forward's
// logsumexp; "Triton-FlashAttention" README, Phase 1 (separate dq and dk/dv
// kernels, masked loads for ragged lengths) and its deferred scope (GQA
// backward accumulates every q head of a group into the shared dK, dV)):
//   P  = exp(scale S - lse)                 (S = Q K^T, lse from the forward)
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  delta = rowsum(dO * O)
//   dQ = scale dS K,  dK = scale dS^T Q    (dK, dV summed over a kv head's group)
//
// gfx950 design, two kernels, no atomics:
//   * bwd_dq: the forward's shape.  A workgroup of 8 waves owns 256 query rows
//     of one q head; it first forms lse * log2(e) and delta for its rows from
//     O and dO and stores them, as (float, float) pairs, for bwd_dkdv.
//     Q and dO are register-resident B operands, K and V tiles
//     of 64 keys stream through a 3-stage LDS ring (buffer-to-LDS loads).
//     S^T = K Q^T and dP^T = V dO^T come out one query per lane, so lse and
//     delta are one value per lane; dQ^T += K^T dS^T reads K^T with the
//     transposing LDS read from the same tile.
//   * bwd_dkdv: the roles swapped.  A workgroup of 8 waves owns 128 keys of
//     one kv head, held in LDS with their V rows; each wave pair shares 32 keys
//     and splits every 64-query tile.  It streams the Q, dO, lse/delta tiles of
//     every q head of the group (2-stage ring), so the group's gradients add
//     up in registers.  S = Q K^T and dP = dO V^T come out one key per lane;
//     dV^T += dO^T P and dK^T += Q^T dS read dO^T and Q^T with the transposing
//     LDS read; the pair's partial sums are added through LDS at the end.
//   The 16-bit P (and dS) B operands take the key (query) order of the fp32
//   accumulator registers, matched by the transposing reads' addresses, as in
//   the forward.  Causal: the dq loop stops at its block's diagonal, the dkdv
//   loop starts at its block's first visible query; only tiles crossing the
//   diagonal are masked.  Ragged tails read as zeros and contribute nothing.
#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "lds_tile.hpp"

namespace attn {

namespace {

constexpr int kDqW = 8;           // waves per dq workgroup (two per SIMD)
constexpr int kDqRows = 32 * kDqW; // query rows per dq workgroup
constexpr int kKvW = 8;           // waves per dkdv workgroup (two per SIMD)
constexpr int kKvRows = 128;      // keys per dkdv workgroup (32 per wave pair)
constexpr int kBT = 64;           // streamed rows per LDS tile
constexpr int kBStages = 3;      // LDS ring depth
// software-pipeline depths: steps of LDS operand reads in flight ahead of the MFMAs that use them
constexpr int kDqReadAhead = 1;    // dQ pass: K/V reads ahead of its S, dP MFMAs
constexpr int kKvReadAhead = 1;    // dK/dV pass: operand reads ahead of its S, dP MFMAs
constexpr int kKvTrReadAhead = 1;  // dK/dV pass: transposing reads ahead of its dV, dK MFMAs

// LDS ring of the dq kernel: V tiles of all stages, then K tiles
template <int D>
struct DqLds {
  static constexpr int TILE = kBT * D;
  static constexpr int V0 = 0;
  static constexpr int K0 = kBStages * TILE;
  static constexpr int ELEMS = 2 * kBStages * TILE;
};

// LDS of the dkdv kernel: the block's K and V rows, a 2-stage ring of (Q, dO)
// tile pairs, and the (lse2, delta) rows of each stage
template <int D>
struct DkvLds {
  static constexpr int TILE = kBT * D;        // one Q (or dO) tile
  static constexpr int KB = kKvRows * D;      // the block's K (or V) rows
  static constexpr int K0 = 0;
  static constexpr int V0 = KB;
  static constexpr int Q0 = 2 * KB;           // stage s: Q at Q0 + 2 s TILE, dO right after
  static constexpr int LD0 = 2 * KB + 2 * 2 * TILE;  // in 16-bit elements; 2 kBT floats per stage
  static constexpr int ELEMS = LD0 + 2 * 4 * kBT;
  static_assert(2 * (2 * 2 * TILE) <= 65536, "Q/dO read offsets fit the 16-bit DS offset");
};

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0; expcnt, lgkmcnt at
// their maxima, i.e. unconstrained)
constexpr int kWaitCnt(int vm) { return 0x0F70 | vm; }

// transposing-read addresses (byte, within stage 0 of a region at `base`) of
// the A operand X^T for an MFMA whose k runs over 16 rows of a row-major tile:
// lane (g = lane/16, i = lane%16) reads row 8u + 4(g/2) + i/4 of the 16-row
// chunk, columns 32dt + 16(g%2) + 4(i%4) .. +3; reads u = 0 / 1 give k-slots
// 0-3 / 4-7, the order in which pack_pt below lays out the B operand
template <int D>
__device__ __forceinline__ void tr_addrs(uint32_t base, int lane, uint32_t (&ad)[D / 32][2]) {
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 8 * u + 4 * (g >> 1) + (i >> 2);
      const int d = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
      ad[dt][u] = opaque_lds(base + 2 * (row * D + ((((d >> 3) ^ swz<D>(row)) << 3) | (d & 7))));
    }
}

// plain-read addresses of the A operand X (rows of the tile, k over columns):
// lane (n = lane%32, hh = lane/32) reads row n, 16-byte chunk 2 ks + hh
template <int D>
__device__ __forceinline__ void row_addrs(uint32_t base, int lane, uint32_t (&ad)[D / 16]) {
  const int n = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) ad[ks] = opaque_lds(base + 2 * (n * D + (((2 * ks + hh) ^ swz<D>(n)) << 3)));
}

// fp32 accumulator x (32x32 tile, element e of lane (n, hh) at row 8(e/4) +
// 4hh + e%4) -> the 16-bit B operands of two MFMA k-steps over those rows:
// pf[kk] holds rows 16kk + 8u + 4hh + t in k-slot 4u + t
template <bool BF16>
__device__ __forceinline__ void pack_pt(const f32x16& x, u32x4* pf) {
#pragma unroll
  for (int e = 0; e < 16; e += 2) pf[e >> 3][(e & 7) >> 1] = pack2<BF16>(x[e], x[e + 1]);
}

// open side of a band: a bound no key or query reaches
constexpr int kOpen = 1 << 30;

// ---- dQ: one workgroup per (batch, q head, 256 query rows).  MASK 0: none;
//      1: causal (j <= i + off); 2: band i + off - win_left <= j <= i + off + win_right
template <int D, bool BF16, int MASK, bool VARLEN>
__global__ __launch_bounds__(64 * kDqW, 2) void bwd_dq_kernel(const BwdArgs a) {
  constexpr bool CAUSAL = MASK == 1, BAND = MASK == 2;
  using L = DqLds<D>;
  constexpr int KS = D / 16, DT = D / 32, C = D / 8;
  constexpr int NB = L::TILE * 2 / 1024 / kDqW;  // 1 KiB DMA blocks per wave per tile
  constexpr int RPB = 64 / C;                   // rows per 1 KiB block
  static_assert(NB >= 1, "every wave loads at least one block");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[L::ELEMS];

  // which (batch, q head, query block): under a causal mask the last blocks
  // see the most keys, so the costliest blocks start first.  With the remap,
  // XCD x (workgroup i runs on XCD i % 8) takes a contiguous span of whole
  // (batch, kv head) units, each unit's blocks query block major and its q
  // heads innermost, so the q heads sharing a kv head stream its K and V
  // tiles together through one L2; otherwise the grid is query block major
  // over all (batch, head) pairs
  int qb, b, h;
  if (!VARLEN && a.dq_remap) {
    const int lid = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int per_unit = a.group * a.nqb;
    const int unit = lid / per_unit, rem = lid - unit * per_unit;
    qb = rem / a.group;
    b = unit / a.Hkv;
    h = (unit - b * a.Hkv) * a.group + (rem - qb * a.group);
  } else {
    const int heads = a.B * a.Hq;
    qb = blockIdx.x / heads;
    const int bh = blockIdx.x - qb * heads;
    b = bh / a.Hq;
    h = bh - b * a.Hq;
  }
  if (MASK != 0) qb = a.nqb - 1 - qb;
  const int kvh = h / a.group;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int q0 = qb * kDqRows;
  const int qrow = q0 + 32 * w + n;

  // ---- this (sequence, head): row counts, first elements, valid bytes.  A
  //      packed sequence's offsets are clamped into the packed tensors; its
  //      query rows are capped at the max_seqlen_q bound (a.Nq)
  int Nq = a.Nq, Nkv = a.Nkv;
  int off = MASK != 0 ? a.causal_off : 0;
  int64_t t0 = 0, s0 = 0;
  int64_t q_bytes = a.q_bytes, do_bytes = a.do_bytes;
  if constexpr (VARLEN) {
    t0 = min(max(a.cu_q[b], 0), a.total_q);
    const int t1 = min(max(a.cu_q[b + 1], (int)t0), a.total_q);
    s0 = min(max(a.cu_k[b], 0), a.total_k);
    const int s1 = min(max(a.cu_k[b + 1], (int)s0), a.total_k);
    Nq = t1 - (int)t0;
    Nkv = s1 - (int)s0;
    if (MASK != 0) off = a.causal_br ? Nkv - Nq : 0;  // from the sequence's own lengths
    Nq = min(Nq, a.Nq);
    if (q0 >= Nq) return;  // whole workgroup
    q_bytes = ((int64_t)(Nq - 1) * a.sqn + D) * 2;
    do_bytes = ((int64_t)(Nq - 1) * a.sdon + D) * 2;
  }
  const int64_t bq = VARLEN ? t0 : 0, bk = VARLEN ? s0 : 0;  // packed: first row of the sequence
  const uint16_t* qbase = a.q + (VARLEN ? bq * a.sqn : (int64_t)b * a.sqb) + (int64_t)h * a.sqh;
  const uint16_t* gbase = a.dout + (VARLEN ? bq * a.sdon : (int64_t)b * a.sdob) + (int64_t)h * a.sdoh;
  const uint16_t* obase = a.o + (VARLEN ? bq * a.son : (int64_t)b * a.sob) + (int64_t)h * a.soh;
  // (lse, delta) rows of this (sequence, q head): (b, h) of (B, Hq, Nq), packed (h, bq) of (Hq, total_q)
  const int64_t row0 = VARLEN ? (int64_t)h * a.total_q + bq : ((int64_t)b * a.Hq + h) * a.Nq;

  // stationary B operands: Q and dO rows (zeros past Nq); the O rows for delta
  u32x4 qf[KS], gf[KS], of[KS];
  {
    const int64_t qo = (int64_t)q0 * a.sqn, go = (int64_t)q0 * a.sdon, oo = (int64_t)q0 * a.son;
    const int64_t o_bytes = ((int64_t)(Nq - 1) * a.son + D) * 2;
    const auto rq = make_rsrc(qbase + qo, clamp_bytes(q_bytes - 2 * qo));
    const auto rg = make_rsrc(gbase + go, clamp_bytes(do_bytes - 2 * go));
    const auto ro = make_rsrc(obase + oo, clamp_bytes(o_bytes - 2 * oo));
    const int32_t oq = (32 * w + n) * (int32_t)a.sqn * 2 + 16 * hh;
    const int32_t og = (32 * w + n) * (int32_t)a.sdon * 2 + 16 * hh;
    const int32_t ob = (32 * w + n) * (int32_t)a.son * 2 + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = bload16(rq, oq + 32 * ks);
      gf[ks] = bload16(rg, og + 32 * ks);
      of[ks] = bload16(ro, ob + 32 * ks);
    }
  }
  float lse2 = 0.f;
  if (qrow < Nq) lse2 = a.lse[row0 + qrow] * kLog2e;
  // wait for these loads here, before the ring's buffer-to-LDS loads go out:
  // the compiler does not see those loads, and a wait it placed at the first
  // use of Q or dO inside the KV loop would also wait, on every tile, for the
  // loads of the tile two ahead
  __builtin_amdgcn_s_waitcnt(kWaitCnt(0));

  // delta = rowsum(dO * O) in fp32: one partial sum per 16-byte chunk (this
  // lane holds chunks 2 ks + hh of row n), chunk pairs added across the two
  // lane halves, then a pairwise tree over the pairs
  float delta;
  {
    float ps[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s += to_f32<BF16>(of[ks][j] & 0xffff) * to_f32<BF16>(gf[ks][j] & 0xffff);
        s += to_f32<BF16>(of[ks][j] >> 16) * to_f32<BF16>(gf[ks][j] >> 16);
      }
      ps[ks] = s + __shfl_xor(s, 32);
    }
#pragma unroll
    for (int m = 1; m < KS; m <<= 1)
#pragma unroll
      for (int i = 0; i < KS; i += 2 * m) ps[i] += ps[i + m];
    delta = ps[0];
  }
  // every query row of the sequence belongs to one dq workgroup, which hands
  // its (lse2, delta) pair to the dK/dV pass (launched after this one)
  if (qrow < Nq) {
    if (hh == 0) reinterpret_cast<float2*>(a.ld)[row0 + qrow] = make_float2(lse2, delta);
  } else {
    delta = 0.f;
  }

  const uint16_t* kbase = a.k + (VARLEN ? bk * a.skn : (int64_t)b * a.skb) + (int64_t)kvh * a.skh;
  const uint16_t* vbase = a.v + (VARLEN ? bk * a.svn : (int64_t)b * a.svb) + (int64_t)kvh * a.svh;
  const int WL = BAND ? (a.win_left < 0 ? kOpen : a.win_left) : 0;
  const int WR = BAND ? (a.win_right < 0 ? kOpen : a.win_right) : 0;
  // keys this block's rows see: up to the diagonal (causal), within the band
  const int kv_end = CAUSAL ? max(0, min(Nkv, q0 + kDqRows + off))
                            : (BAND ? max(0, min(Nkv, q0 + kDqRows + off + WR)) : Nkv);
  const int ntiles = (kv_end + kBT - 1) / kBT;
  const int t_begin = BAND ? min(max(0, q0 + off - WL) / kBT, ntiles) : 0;
  // tiles every row sees in full: [full_lo, n_full)
  const int n_full = CAUSAL ? max(0, min(q0 + off + 1, Nkv)) / kBT
                            : (BAND ? max(0, min(Nkv, q0 + off + WR + 1)) / kBT : Nkv / kBT);
  const int full_lo = BAND ? (max(0, q0 + kDqRows - 1 + off - WL) + kBT - 1) / kBT : 0;

  // DMA geometry (as the forward): wave w fills 1 KiB blocks NB w .. NB w + NB - 1
  int32_t dk[NB], dv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = RPB * (NB * w + i) + lane / C;
    const int chunk = (lane % C) ^ swz<D>(row);
    dk[i] = row * (int32_t)a.skn * 2 + 16 * chunk;
    dv[i] = row * (int32_t)a.svn * 2 + 16 * chunk;
  }
  const uint32_t lds_k = lds_addr(smem + L::K0) + 1024 * NB * w;
  const uint32_t lds_v = lds_addr(smem + L::V0) + 1024 * NB * w;
  auto dma_tile = [&](int t, int stage) __attribute__((always_inline)) {
    const int64_t ko = (int64_t)t * kBT * a.skn, vo = (int64_t)t * kBT * a.svn;
    // each load's range ends with the tile's last key row (none past Nkv)
    const int rows = min(Nkv - t * kBT, kBT);
    const i32x4 rk = rsrc_words(kbase + ko, rows > 0 ? ((rows - 1) * (int32_t)a.skn + D) * 2 : 0);
    const i32x4 rv = rsrc_words(vbase + vo, rows > 0 ? ((rows - 1) * (int32_t)a.svn + D) * 2 : 0);
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(rk, lds_k + 2 * stage * L::TILE + 1024 * i, dk[i]);
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(rv, lds_v + 2 * stage * L::TILE + 1024 * i, dv[i]);
  };

  uint32_t ka[KS], va[KS], kt[DT][2];
  row_addrs<D>(lds_addr(smem + L::K0), lane, ka);
  row_addrs<D>(lds_addr(smem + L::V0), lane, va);
  tr_addrs<D>(lds_addr(smem + L::K0), lane, kt);

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  const float c = a.c;
  const int wq_hi = q0 + 32 * w + 31 + off;
  const int wq_lo = q0 + 32 * w + off;

  // the stage and whether the tile needs masks are compile-time, so the
  // stage offsets fold into the LDS reads' immediate offsets and full tiles
  // carry no mask arithmetic
  auto compute = [&](auto stage_tag, int t, bool masked) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;
    const int kb = t * kBT;
    bool act1 = true;
    if (masked) {
      if (kb >= Nkv || (CAUSAL && kb > wq_hi)) return;
      if (BAND && (kb > wq_hi + WR || kb + kBT - 1 < wq_lo - WL)) return;  // outside this wave's band
      act1 = kb + 32 < Nkv && (!CAUSAL || kb + 32 <= wq_hi) && (!BAND || kb + 32 <= wq_hi + WR);
    }
    // per 32-key subtile u: S^T = K Q^T, dP^T = V dO^T, then dS^T = P^T (dP^T -
    // delta) with P^T = exp2(S^T c - lse2); element e of lane (n, hh) is key
    // kb + 32u + 8(e/4) + 4hh + e%4
    u32x4 pf[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !act1) break;
      const uint32_t so = 2 * stage * L::TILE + 2 * 32 * u * D;
      f32x16 sx = f32x16{}, px = f32x16{};
      {
        // software pipeline: k-step ks + PF's K and V reads go out before
        // k-step ks's two MFMAs; the fences keep them there
        constexpr int PF = kDqReadAhead;
        u32x4 opk[PF + 1], opv[PF + 1];
        auto issue = [&](int ks) __attribute__((always_inline)) {
          opk[ks % (PF + 1)] = lds_load16(ka[ks] + so);
          opv[ks % (PF + 1)] = lds_load16(va[ks] + so);
        };
#pragma unroll
        for (int ks = 0; ks < PF; ++ks) issue(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + PF < KS) issue(ks + PF);
          __builtin_amdgcn_sched_barrier(0);
          sx = mfma_32x32x16<BF16>(opk[ks % (PF + 1)], qf[ks], sx);
          px = mfma_32x32x16<BF16>(opv[ks % (PF + 1)], gf[ks], px);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the mask test sits outside the element loop: inside it the compiler
      // branched on it once per element
      auto soft = [&](auto mask_tag) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float pv = fast_exp2(__builtin_fmaf(sx[e], c, -lse2));
          if constexpr (decltype(mask_tag)::value) {
            const int key = kb + 32 * u + 8 * (e >> 2) + 4 * hh + (e & 3);
            pv = (key < Nkv && (!CAUSAL || key <= qrow + off) &&
                  (!BAND || (key >= qrow + off - WL && key <= qrow + off + WR))) ? pv : 0.f;
          }
          sx[e] = pv * (px[e] - delta);
        }
      };
      if (masked)
        soft(std::true_type{});
      else
        soft(std::false_type{});
      pack_pt<BF16>(sx, pf + 2 * u);
    }
    const uint32_t so = 2 * stage * L::TILE;
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 2 || act1) {
        const uint32_t o = so + 2 * 16 * kk * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x2 lo = lds_read_tr16(kt[dt][0] + o);
          const u32x2 hi = lds_read_tr16(kt[dt][1] + o);
          acc[dt] = mfma_32x32x16<BF16>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kk], acc[dt]);
        }
      }
    }
  };

  // 3-stage ring: the loads of tile t + 2 go out before tile t is computed
  constexpr int NDMA = 2 * NB;
  static_assert(NDMA < 16, "vmcnt field");
  if (t_begin < ntiles) dma_tile(t_begin, 0);
  if (t_begin + 1 < ntiles) dma_tile(t_begin + 1, 1);
  if (t_begin + 1 < ntiles)
    __builtin_amdgcn_s_waitcnt(kWaitCnt(NDMA));
  else
    __builtin_amdgcn_s_waitcnt(kWaitCnt(0));
  barrier_nofence();
  // tile t sits in stage (t - t_begin) % 3: the loop steps through the three
  // stages with the stage a compile-time constant
  auto step = [&](int t, auto stage_tag) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;
    const bool pre = t + 2 < ntiles;
    if (pre) dma_tile(t + 2, (stage + 2) % 3);
    compute(stage_tag, t, t >= n_full || t < full_lo);
    if (pre)
      __builtin_amdgcn_s_waitcnt(kWaitCnt(NDMA));
    else
      __builtin_amdgcn_s_waitcnt(kWaitCnt(0));
    barrier_nofence();
  };
  int t = t_begin;
  for (; t + 2 < ntiles; t += 3) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
    step(t + 2, std::integral_constant<int, 2>{});
  }
  if (t < ntiles) step(t, std::integral_constant<int, 0>{});
  if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});

  // ---- dQ = scale (dQ^T)^T, cast, stored as whole rows through the wave's
  //      slice of the ring (every wave is past the last barrier)
  uint16_t* const dqb = a.dq + (VARLEN ? bq * a.sdqn : (int64_t)b * a.sdqb) + (int64_t)h * a.sdqh;
  static_assert(kDqW * 32 * 2 * D <= L::ELEMS * 2, "every wave's rows fit in the ring");
  store_tile_rows<D, BF16>(lds_addr(smem) + w * 32 * 2 * D, acc, a.scale, dqb, a.sdqn, q0 + 32 * w, Nq);
}

// ---- dK, dV: one workgroup per (batch, kv head, 128 keys).  Wave w owns keys
//      32 (w % 4) .. +31 and, of every 64-query tile, the 32 queries
//      32 (w / 4) .. +31; the two waves of a key group add their partial dK,
//      dV through LDS at the end.  The block's K and V rows sit in LDS (B
//      operands read with plain 16-byte reads), so only the two accumulators
//      are register-resident and two waves fit on each SIMD.
template <int D, bool BF16, int MASK, bool VARLEN>
__global__ __launch_bounds__(64 * kKvW, 2) void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr bool CAUSAL = MASK == 1, BAND = MASK == 2;
  using L = DkvLds<D>;
  constexpr int KS = D / 16, DT = D / 32, C = D / 8;
  constexpr int NB = L::TILE * 2 / 1024 / kKvW;   // 1 KiB DMA blocks per wave per Q (dO) tile
  constexpr int NBK = L::KB * 2 / 1024 / kKvW;    // ... per K (V) block
  constexpr int RPB = 64 / C;
  static_assert(NB >= 1 && NBK >= 1, "every wave loads at least one block");
  // the partial sums of the kKvW / 2 second-half waves (2 accumulators x DT x
  // 16 floats x 64 lanes) fit in the LDS they reuse
  static_assert((kKvW / 2) * 2 * DT * 16 * 64 * 4 <= L::ELEMS * 2, "partial sums fit in LDS");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[L::ELEMS];

  // which (batch, kv head, key block): under a causal mask the first blocks
  // see the most queries, so the costliest blocks start first.  With the
  // remap, XCD x (workgroup i runs on XCD i % 8) takes a contiguous span of
  // whole units, so a unit's key blocks run together on one XCD; otherwise
  // the grid is key block major over all units
  int kbk, unit;
  if (!VARLEN && a.dkv_remap) {
    const int lid = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    unit = lid / a.nkb;
    kbk = lid - unit * a.nkb;
  } else {
    const int units = a.B * a.Hkv;
    kbk = blockIdx.x / units;
    unit = blockIdx.x - kbk * units;
  }
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w & 3, qh = w >> 2;  // key group, query half
  const int n = lane & 31, hh = lane >> 5;
  const int k0 = kbk * kKvRows;
  const int key = k0 + 32 * kg + n;

  // ---- this (sequence, kv head): row counts, first rows, valid bytes (as in
  //      the dQ pass; a.Nq, a.Nkv are the max_seqlen bounds when packed)
  int Nq = a.Nq, Nkv = a.Nkv;
  int off = MASK != 0 ? a.causal_off : 0;
  int64_t bq = 0, bk = 0;
  int64_t k_bytes = a.k_bytes, v_bytes = a.v_bytes;
  if constexpr (VARLEN) {
    bq = min(max(a.cu_q[b], 0), a.total_q);
    const int t1 = min(max(a.cu_q[b + 1], (int)bq), a.total_q);
    bk = min(max(a.cu_k[b], 0), a.total_k);
    const int s1 = min(max(a.cu_k[b + 1], (int)bk), a.total_k);
    Nq = t1 - (int)bq;
    Nkv = s1 - (int)bk;
    if (MASK != 0) off = a.causal_br ? Nkv - Nq : 0;
    Nq = min(Nq, a.Nq);
    if (k0 >= Nkv) return;  // whole workgroup: block past this sequence's keys
    k_bytes = ((int64_t)(Nkv - 1) * a.skn + D) * 2;
    v_bytes = ((int64_t)(Nkv - 1) * a.svn + D) * 2;
  }
  const uint16_t* kbase = a.k + (VARLEN ? bk * a.skn : (int64_t)b * a.skb) + (int64_t)kvh * a.skh;
  const uint16_t* vbase = a.v + (VARLEN ? bk * a.svn : (int64_t)b * a.svb) + (int64_t)kvh * a.svh;

  // query tiles that see some key of the block, for every q head of the
  // group: query i sees key j iff j <= i + off (causal), iff i + off - WL <=
  // j <= i + off + WR (band); tiles in [full_lo, full_hi) see every key of it
  const int WL = BAND ? (a.win_left < 0 ? kOpen : a.win_left) : 0;
  const int WR = BAND ? (a.win_right < 0 ? kOpen : a.win_right) : 0;
  const int ntq0 = (Nq + kBT - 1) / kBT;
  const int ntq = BAND ? min(ntq0, (max(0, min(Nq, k0 + kKvRows - off + WL)) + kBT - 1) / kBT) : ntq0;
  const int tq0 = CAUSAL ? min(max(0, k0 - off) / kBT, ntq)
                         : (BAND ? min(max(0, k0 - off - WR) / kBT, ntq) : 0);
  const int full_lo = CAUSAL ? min(ntq, (max(0, k0 + kKvRows - 1 - off) + kBT - 1) / kBT)
                             : (BAND ? (max(0, k0 + kKvRows - 1 - off - WR) + kBT - 1) / kBT : 0);
  const int full_hi = BAND ? max(0, k0 - off + WL + 1) / kBT : ntq;
  const int nt = ntq - tq0;
  const int total = nt * a.group;

  // DMA: the block's K and V rows once, then per tile the Q and dO rows and
  // the (lse2, delta) pairs (8 bytes a row, 64 bytes a wave, 4 lanes: a
  // buffer-to-LDS load writes for every active lane)
  auto dma_rows = [&](int32_t (&o)[NBK], int64_t stride) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int row = RPB * (NBK * w + i) + lane / C;
      o[i] = row * (int32_t)stride * 2 + 16 * ((lane % C) ^ swz<D>(row));
    }
  };
  {
    int32_t ok[NBK], ov[NBK];
    dma_rows(ok, a.skn);
    dma_rows(ov, a.svn);
    const int64_t ko = (int64_t)k0 * a.skn, vo = (int64_t)k0 * a.svn;
    const i32x4 rk = rsrc_words(kbase + ko, clamp_bytes(k_bytes - 2 * ko));
    const i32x4 rv = rsrc_words(vbase + vo, clamp_bytes(v_bytes - 2 * vo));
#pragma unroll
    for (int i = 0; i < NBK; ++i) dma16(rk, lds_addr(smem + L::K0) + 1024 * (NBK * w + i), ok[i]);
#pragma unroll
    for (int i = 0; i < NBK; ++i) dma16(rv, lds_addr(smem + L::V0) + 1024 * (NBK * w + i), ov[i]);
  }
  int32_t dq_[NB], dg_[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = RPB * (NB * w + i) + lane / C;
    const int chunk = (lane % C) ^ swz<D>(row);
    dq_[i] = row * (int32_t)a.sqn * 2 + 16 * chunk;
    dg_[i] = row * (int32_t)a.sdon * 2 + 16 * chunk;
  }
  constexpr int LDW = kBT * 8 / kKvW;  // (lse2, delta) bytes per wave per tile
  const uint32_t lds_q = lds_addr(smem + L::Q0) + 1024 * NB * w;
  const uint32_t lds_ld = lds_addr(smem + L::LD0) + LDW * w;
  // (lse2, delta) row 0 of q head h: (b, h) of (B, Hq, Nq), packed (h, bq) of (Hq, total_q)
  auto ld_row0 = [&](int h) __attribute__((always_inline)) {
    return a.ld + 2 * (VARLEN ? (int64_t)h * a.total_q + bq : ((int64_t)b * a.Hq + h) * a.Nq);
  };
  // step it takes query tile ntq - 1 - it / group of q head it % group: the
  // last tile first and the group's q heads innermost, so the key blocks of
  // one (batch, kv head) running together read the same Q and dO tiles at
  // the same time (every block's range ends at the last tile)
  // byte addresses of the first Q, dO and (lse2, delta) row of query tile t
  // of q head kvh * group + hg, and the steps from one tile of the walk to the
  // next: the next q head, or from the group's last q head back to its first
  // one tile lower.  Each load's range ends with the tile's last row.
  const int64_t lstride = 8 * (VARLEN ? (int64_t)a.total_q : (int64_t)a.Nq);  // between q heads
  const int64_t gm1 = a.group - 1;
  const int64_t sq_h = 2 * a.sqh, sq_w = -gm1 * 2 * a.sqh - 2 * kBT * a.sqn;
  const int64_t sg_h = 2 * a.sdoh, sg_w = -gm1 * 2 * a.sdoh - 2 * kBT * a.sdon;
  const int64_t sl_h = lstride, sl_w = -gm1 * lstride - 8 * kBT;
  auto dma_tile = [&](int t, uint64_t aq, uint64_t ag, uint64_t al, int stage) __attribute__((always_inline)) {
    const int rows = min(Nq - t * kBT, kBT);  // >= 1: t < ntq
    const i32x4 rq = rsrc_words((const void*)aq, ((rows - 1) * (int32_t)a.sqn + D) * 2);
    const i32x4 rg = rsrc_words((const void*)ag, ((rows - 1) * (int32_t)a.sdon + D) * 2);
    const i32x4 rl = rsrc_words((const void*)al, rows * 8);
    const uint32_t sq = lds_q + stage * 2 * L::TILE * 2;
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(rq, sq + 1024 * i, dq_[i]);
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(rg, sq + 2 * L::TILE + 1024 * i, dg_[i]);
    if (lane < LDW / 16) dma16(rl, lds_ld + stage * 4 * kBT * 2, LDW * w + 16 * lane);
  };

  // LDS operand addresses; Q-tile addresses reach the dO tile, the other
  // stage and the subtiles through immediate offsets (< 64 KiB), and the K
  // addresses reach V the same way
  uint32_t qa[KS], qt[DT][2], kva[KS];
  row_addrs<D>(lds_addr(smem + L::Q0) + 2 * 32 * qh * D, lane, qa);
  tr_addrs<D>(lds_addr(smem + L::Q0) + 2 * 32 * qh * D, lane, qt);
  row_addrs<D>(lds_addr(smem + L::K0) + 2 * 32 * kg * D, lane, kva);
  const uint32_t ldr = opaque_lds(lds_addr(smem + L::LD0) + 32 * qh * 8 + 32 * hh);  // + 8g * 8 per read

  f32x16 adv[DT], adk[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    adv[dt] = f32x16{};
    adk[dt] = f32x16{};
  }
  const float c = a.c;
  const int kmin = k0 + 32 * kg;  // this wave's first key

  // the stage and whether the tile needs masks are compile-time (as in the
  // dQ pass)
  auto compute = [&](auto stage_tag, int t, bool masked) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;
    const int tq = t * kBT + 32 * qh;  // this wave's first query
    // 32 queries that see none of this wave's keys
    if (masked && CAUSAL && kmin > tq + 31 + off) return;
    if (masked && BAND && (kmin > tq + 31 + off + WR || kmin + 31 < tq + off - WL)) return;
    constexpr uint32_t sq = stage * 2 * L::TILE * 2, sg = sq + 2 * L::TILE;
    f32x16 sx = f32x16{}, px = f32x16{};
    // software pipeline: the four operand reads of k-step ks + PF go out before
    // k-step ks's two MFMAs (a loaded LDS read takes some 250 cycles); the
    // scheduling fences keep the compiler from sinking them next to their use
    constexpr int PF = kKvReadAhead;
    u32x4 opq[PF + 1], opk[PF + 1], opg[PF + 1], opv[PF + 1];
    auto issue = [&](int ks) __attribute__((always_inline)) {
      const int r = ks % (PF + 1);
      opq[r] = lds_load16(qa[ks] + sq);
      opk[r] = lds_load16(kva[ks]);
      opg[r] = lds_load16(qa[ks] + sg);
      opv[r] = lds_load16(kva[ks] + 2 * L::KB);
    };
    // the (lse2, delta) pairs of this wave's 16 queries per lane, read with the
    // last k-step's MFMAs in flight
    f32x4 ldp[8];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) issue(ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) issue(ks + PF);
      if (ks == KS - 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          ldp[i] = __builtin_bit_cast(f32x4, lds_load16(ldr + stage * 4 * kBT * 2 + 8 * (i >> 1) * 8 + 16 * (i & 1)));
      }
      __builtin_amdgcn_sched_barrier(0);
      const int r = ks % (PF + 1);
      sx = mfma_32x32x16<BF16>(opq[r], opk[r], sx);
      px = mfma_32x32x16<BF16>(opg[r], opv[r], px);
      __builtin_amdgcn_sched_barrier(0);
    }
    // element e of lane (n, hh) is query tq + 8(e/4) + 4hh + e%4, key `key`
    // the mask test sits outside the element loop (as in the dQ pass)
    auto soft = [&](auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MK = decltype(mask_tag)::value;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a0 = ldp[2 * g], a1 = ldp[2 * g + 1];
        const float l2[4] = {a0[0], a0[2], a1[0], a1[2]};
        const float dl[4] = {a0[1], a0[3], a1[1], a1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * g + j;
          float pv = fast_exp2(__builtin_fmaf(sx[e], c, -l2[j]));
          if constexpr (MK && CAUSAL) pv = (key <= tq + 8 * g + 4 * hh + j + off) ? pv : 0.f;
          if constexpr (MK && BAND) {
            const int p = tq + 8 * g + 4 * hh + j + off;
            pv = (key >= p - WL && key <= p + WR) ? pv : 0.f;
          }
          sx[e] = pv;
          px[e] = pv * (px[e] - dl[j]);
        }
      }
    };
    if (masked)
      soft(std::true_type{});
    else
      soft(std::false_type{});
    u32x4 pp[2], dp[2];
    pack_pt<BF16>(sx, pp);
    pack_pt<BF16>(px, dp);
    // dV^T += dO^T P and dK^T += Q^T dS over this wave's 32 queries
    {
      // the same software pipeline over the 2 x DT steps (kk, dt), four
      // transposing reads a step
      constexpr int GP = kKvTrReadAhead, NS = 2 * DT;
      u32x4 opg[GP + 1], opq[GP + 1];
      auto issue = [&](int i) __attribute__((always_inline)) {
        const int r = i % (GP + 1), kk = i / DT, dt = i % DT;
        const uint32_t o = sq + 2 * 16 * kk * D;
        const u32x2 glo = lds_read_tr16(qt[dt][0] + o + 2 * L::TILE);
        const u32x2 ghi = lds_read_tr16(qt[dt][1] + o + 2 * L::TILE);
        const u32x2 qlo = lds_read_tr16(qt[dt][0] + o);
        const u32x2 qhi = lds_read_tr16(qt[dt][1] + o);
        opg[r] = u32x4{glo[0], glo[1], ghi[0], ghi[1]};
        opq[r] = u32x4{qlo[0], qlo[1], qhi[0], qhi[1]};
      };
#pragma unroll
      for (int i = 0; i < GP; ++i) issue(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + GP < NS) issue(i + GP);
        __builtin_amdgcn_sched_barrier(0);
        const int r = i % (GP + 1), kk = i / DT, dt = i % DT;
        adv[dt] = mfma_32x32x16<BF16>(opg[r], pp[kk], adv[dt]);
        adk[dt] = mfma_32x32x16<BF16>(opq[r], dp[kk], adk[dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // 2-stage ring: the loads of tile it + 1 go out before tile it is computed
  // (t, hg) and the addresses of step it, counted along the walk
  int t = ntq - 1, hg = 0;
  const int64_t h0 = (int64_t)kvh * a.group, r0 = (int64_t)(ntq - 1) * kBT;
  uint64_t aq = (uint64_t)a.q + 2 * ((VARLEN ? bq * a.sqn : (int64_t)b * a.sqb) + h0 * a.sqh + r0 * a.sqn);
  uint64_t ag = (uint64_t)a.dout + 2 * ((VARLEN ? bq * a.sdon : (int64_t)b * a.sdob) + h0 * a.sdoh + r0 * a.sdon);
  uint64_t al = (uint64_t)ld_row0((int)h0) + 8 * r0;
  if (total > 0) dma_tile(t, aq, ag, al, 0);
  __builtin_amdgcn_s_waitcnt(kWaitCnt(0));
  barrier_nofence();
  auto step = [&](int it, auto stage_tag) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;
    int tn = t, hn = hg + 1;
    const bool wrap = hn == a.group;
    if (wrap) {
      hn = 0;
      --tn;
    }
    const uint64_t aqn = aq + (uint64_t)(wrap ? sq_w : sq_h), agn = ag + (uint64_t)(wrap ? sg_w : sg_h),
                   aln = al + (uint64_t)(wrap ? sl_w : sl_h);
    if (it + 1 < total) dma_tile(tn, aqn, agn, aln, stage ^ 1);
    compute(stage_tag, t, (MASK != 0) && (t < full_lo || t >= full_hi));
    __builtin_amdgcn_s_waitcnt(kWaitCnt(0));
    barrier_nofence();
    t = tn;
    hg = hn;
    aq = aqn;
    ag = agn;
    al = aln;
  };
  int it = 0;
  for (; it + 1 < total; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    step(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < total) step(it, std::integral_constant<int, 0>{});

  // ---- add the two query halves' partial sums (through LDS), then
  //      dV = (dV^T)^T, dK = scale (dK^T)^T, cast, store
  float* red = reinterpret_cast<float*>(smem);  // [key group][dV, dK][dt][e][lane]
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[(((kg * 2 + 0) * DT + dt) * 16 + e) * 64 + lane] = adv[dt][e];
        red[(((kg * 2 + 1) * DT + dt) * 16 + e) * 64 + lane] = adk[dt][e];
      }
  }
  __syncthreads();
  if (qh == 1 || key >= Nkv) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      adv[dt][e] += red[(((kg * 2 + 0) * DT + dt) * 16 + e) * 64 + lane];
      adk[dt][e] += red[(((kg * 2 + 1) * DT + dt) * 16 + e) * 64 + lane];
    }
  uint16_t* vp = a.dv + (VARLEN ? bk * a.sdvn : (int64_t)b * a.sdvb) + (int64_t)kvh * a.sdvh + (int64_t)key * a.sdvn;
  uint16_t* kp = a.dk + (VARLEN ? bk * a.sdkn : (int64_t)b * a.sdkb) + (int64_t)kvh * a.sdkh + (int64_t)key * a.sdkn;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * hh;
      *reinterpret_cast<u32x2*>(vp + d) = u32x2{pack2<BF16>(adv[dt][4 * g], adv[dt][4 * g + 1]),
                                                pack2<BF16>(adv[dt][4 * g + 2], adv[dt][4 * g + 3])};
      *reinterpret_cast<u32x2*>(kp + d) =
          u32x2{pack2<BF16>(adk[dt][4 * g] * a.scale, adk[dt][4 * g + 1] * a.scale),
                pack2<BF16>(adk[dt][4 * g + 2] * a.scale, adk[dt][4 * g + 3] * a.scale)};
    }
}

template <int D, bool BF16, int MASK, bool VARLEN>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, MASK, VARLEN>), dim3(a.dq_blocks), dim3(64 * kDqW), 0, stream, a);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, BF16, MASK, VARLEN>), dim3(a.dkv_blocks), dim3(64 * kKvW), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool VARLEN>
hipError_t launch_bwd_v(const BwdArgs& a, hipStream_t stream) {
  if (a.mask == 2) return launch_bwd_t<D, BF16, 2, VARLEN>(a, stream);
  return a.mask == 1 ? launch_bwd_t<D, BF16, 1, VARLEN>(a, stream) : launch_bwd_t<D, BF16, 0, VARLEN>(a, stream);
}

template <int D, bool BF16>
hipError_t launch_bwd_m(const BwdArgs& a, hipStream_t stream) {
  return a.cu_q ? launch_bwd_v<D, BF16, true>(a, stream) : launch_bwd_v<D, BF16, false>(a, stream);
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_bwd_m<D, true>(a, stream) : launch_bwd_m<D, false>(a, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, hipStream_t stream) {
  return D == 64 ? launch_bwd_d<64>(a, stream) : launch_bwd_d<128>(a, stream);
}

}  // namespace attn
