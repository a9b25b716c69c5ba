// Fused attention forward (prefill) for gfx950.
//
// What it computes: O = softmax(scale * Q K^T + mask) V and lse, following the
// tiled online-softmax method of "Skill: Write a Triton Attention Kernel"
// (Required reasoning process, steps 1-9) and "FlashAttention Kernel
// Optimization" (Online Softmax; Tiled Computation; Causal Masking), with GQA
// head sharing as in the "Triton-FlashAttention" README (GQA phase).
//
// gfx950 design (not the pages' Triton tiling):
//   * one workgroup = 8 wave64s = 256 query rows of one q head; each wave owns
//     32 rows for the whole KV loop (two waves per SIMD).  Dense grids that
//     256-row blocks would leave at least half empty use 128-row blocks of two
//     (D = 128) or three (D = 64) key groups (below).  Packed batches of
//     short sequences use 128-row blocks of 4 waves and one key group, two
//     workgroups per CU, with bitwise the same per-row arithmetic as 256-row
//     blocks.
//   * KV tiles of 64 rows go from HBM/L2 straight into LDS with buffer-to-LDS
//     loads (no register staging), through a 4-stage ring, row-major with an
//     XOR swizzle of 16-byte slots that keeps every access pattern free of bank
//     conflicts.  The loads of tile t+3 are issued before tile t is computed;
//     the buffer range check writes zeros past the last key, so ragged tails
//     need no branches.  Unmasked grids keep the ring with a barrier per
//     tile; band grids with counters in LDS, and causal ones with counters on
//     their diagonal tiles: there the waves of a block have unequal work and
//     need not wait for each other on every tile.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//     Q is the register-resident B operand and each lane ends up owning one
//     query row's scores.  The P.V MFMA takes V^T as its A operand, assembled
//     by ds_read_b64_tr_b16 (the gfx950 transposing LDS read) from the
//     row-major tile; its key order matches the fp32 score registers, which
//     therefore are directly the B operand: no shuffles between the two
//     contractions.
//   * online softmax in the log2 domain: t = s * scale * log2(e); lanes l and
//     l+32 hold the two halves of a row, and their maxima are exchanged only
//     when the reference max moves (below); the row sum l is accumulated from
//     the fp32 P, which then goes to 16 bits (round to nearest even) right
//     before the P.V MFMA; m, l and O stay fp32.
//   * P is formed against the current reference max first; the reference
//     moves -- rescaling O and l by alpha, P formed again -- only when a
//     row has none yet or a half row's P summed to more than 2^10 on the
//     tile, so the common path forms no row max at all.  O and l are always
//     relative to the same reference, so O / l is unchanged (the rescale of
//     step 5f is an identity); P stays <= 2^10, well inside fp16/bf16 range.
//   * the epilogue stores O as whole rows, through LDS: a lane holds half of
//     its row's columns, which stored directly would touch 32 rows per store.
//   * causal: the KV loop stops at the block's diagonal; tiles below every
//     row's diagonal take a path with no per-element compare, and on the last
//     tiles each wave skips 32-key subtiles that lie wholly above its rows.
//     The diagonal may be shifted (query i sees keys j <= i + off): off = 0 is
//     the pages' top-left mask, off = Nkv - Nq aligns it bottom-right (a chunk
//     of queries at the end of a longer sequence, as in chunked prefill).
#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "lds_tile.hpp"

namespace attn {

namespace {

constexpr int kBN = 64;              // key rows per LDS tile
constexpr float kSumBound = 1024.f;  // lazy rescale: bound on a half row's P sum per tile
// instruction order hints of a tile's two MFMA phases
constexpr int kKLead = 4;   // K fragment reads issued before the first score MFMA
constexpr int kVLead = 2;   // V^T fragments (2 reads each) issued before the first P.V MFMA
constexpr int kValu0 = 40;  // softmax vector instructions before the first P.V MFMA
constexpr int kValu1 = 5;   // softmax vector instructions after each P.V MFMA

// One LDS ring of STAGES (K, V) tile pairs: the V tiles of all stages first,
// then the K tiles, so that every V^T read is its wave's base address plus an
// immediate below 64 KiB
template <int D, int STAGES>
struct PrefillLds {
  static constexpr int C = D / 8;        // 16-byte slots per K/V row
  static constexpr int TILE = kBN * D;   // elements of one K (or V) tile
  static constexpr int V0 = 0;           // V tile of stage s at V0 + s * TILE
  static constexpr int K0 = STAGES * TILE;
  static constexpr int ELEMS = 2 * STAGES * TILE;
  static_assert(2 * (STAGES * TILE) <= 65536, "V^T read offsets fit the 16-bit DS offset");
};

// ring depth: four stages (loads of tile t+3 issued before tile t); two for
// D = 128 tiles in a 4-row-wave workgroup: with two key groups (two rings;
// four stages would need 256 KiB of LDS), or with one, whose 64 KiB ring lets
// two such workgroups share a CU; and two for three key groups (three rings)
template <int D, int KVS, int RW>
constexpr int prefill_stages() {
  return ((D == 128 && RW == 4) || KVS == 3) ? 2 : 4;
}

// MASK 0: every key below Nkv; 1: causal (j <= i + off); 2: a band of keys
// i + off - win_left <= j <= i + off + win_right (either side may be open).
// RW: row waves, 32 query rows each (RW = 8: 256-row blocks; RW = 4: 128).
// KVS: key groups.  With KVS = 2 (3) a workgroup of 8 (12) waves owns 128
// rows; waves w, w + 4 (and w + 8) share a SIMD and the same 32 rows, and each
// streams every second (third) key tile of the block's range through a ring
// of its own, so a grid too small to fill the chip with 256-row blocks still
// runs two (three) waves per SIMD.  The groups' (m, l, O) meet in LDS at the
// end and are merged with the rescale identity of the online softmax.  Three
// groups are used at D = 64, whose kernel fits in the 168 VGPRs that three
// waves per SIMD leave.
template <int D, bool BF16, int MASK, bool VARLEN, int RW, int KVS>
__global__ __launch_bounds__(64 * RW * KVS) __attribute__((amdgpu_waves_per_eu(KVS == 3 ? 3 : 2)))
void prefill_fwd_kernel(const FwdArgs a) {
  constexpr int kWaves = RW * KVS;    // waves per workgroup
  constexpr int kBM = 32 * RW;        // query rows per workgroup
  constexpr int kStages = prefill_stages<D, KVS, RW>();
  static_assert(kStages == 2 || kStages == 4, "the KV loop cycles two or four stages");
  static_assert(KVS >= 1 && KVS <= 3, "one to three key groups");
  constexpr bool CAUSAL = MASK == 1;
  constexpr bool BAND = MASK == 2;
  using L = PrefillLds<D, kStages>;
  constexpr int KS = D / 16;        // k-steps of the score MFMA
  constexpr int DT = D / 32;        // 32-wide head-dim tiles of O
  constexpr int NB = L::C / RW;     // 1 KiB DMA blocks per wave per K (or V) tile
  static_assert(NB >= 1, "every wave loads at least one block");
  constexpr int RPB = 64 / L::C;    // rows per 1 KiB block
  __shared__ __attribute__((aligned(1024))) uint16_t smem[KVS * L::ELEMS];
  // masked grids with one key group and four stages keep the ring with
  // counters in LDS instead of a barrier per tile (KV loop below)
  constexpr bool kCounted = KVS == 1 && kStages == 4 && MASK != 0;
  __shared__ uint32_t ring_cnt[9];
  if constexpr (kCounted) {
    if (threadIdx.x < 9) ring_cnt[threadIdx.x] = 0;
    __syncthreads();
  }

  // ---- which (batch, q head, query block) this workgroup owns
  const int bid = blockIdx.x;
  const int per_unit = a.group * a.nqb;
  int unit, rem;
  if constexpr (VARLEN) {
    // (batch, kv head) units dealt round-robin to the 8 XCDs (workgroup i
    // runs on XCD i % 8), each unit's blocks on one XCD, latest query block
    // first: with Hkv a multiple of 8 every XCD holds the same kv head of
    // every sequence, so the XCDs stay balanced whatever the lengths.
    // (Ordering an XCD's blocks by query-block rank across all its units
    // measured no faster.)
    const int r = (bid >> 3) / per_unit;
    unit = (bid & 7) + 8 * r;
    rem = (bid >> 3) - r * per_unit;
    if (unit >= a.units) return;  // whole workgroup: the grid rounds units up to 8
  } else {
    int lid = bid;
    if (a.remap) lid = (bid & 7) * (a.nblocks >> 3) + (bid >> 3);  // keep a kv head's blocks on one XCD
    unit = lid / per_unit;
    rem = lid - unit * per_unit;
  }
  int qb = rem / a.group;
  const int hg = rem - qb * a.group;
  if (MASK != 0) qb = a.nqb - 1 - qb;  // longest (latest) query blocks first
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int h = kvh * a.group + hg;  // q heads [kvh*group, (kvh+1)*group) share kv head kvh

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave 0..kWaves-1 (uniform)
  // row wave: rows 32 w .. 32 w + 31 of the block.  Waves wv and wv + 4 share
  // a SIMD; in 256-row blocks they take row slices wv and 7 - wv, so that on
  // diagonal and band-edge tiles, where a slice's work grows (or shrinks) with
  // its rank, every SIMD holds the same total
  const int w = KVS == 1 ? (RW == 8 ? (wv < 4 ? wv : 11 - wv) : wv) : wv % RW;
  const int grp = KVS == 1 ? 0 : wv / RW;  // key group
  const int n = lane & 31;   // this lane's query column within the wave
  const int hh = lane >> 5;  // which half of the wave
  const int q0 = qb * kBM;
  const int qrow = q0 + 32 * w + n;

  // ---- this (batch, head) slice: its rows, first elements and valid bytes.
  //      A packed sequence's offsets are clamped into [previous offset, total],
  //      so no access leaves the packed tensors whatever the offsets hold.
  int Nq = a.Nq, Nkv = a.Nkv;
  int off = MASK != 0 ? a.causal_off : 0;
  const uint16_t *qbase, *kbase, *vbase;
  uint16_t* obase;
  float* lbase;
  int64_t q_bytes = a.q_bytes;
  if constexpr (VARLEN) {
    const int t0 = min(max(a.cu_q[b], 0), a.total_q);
    const int t1 = min(max(a.cu_q[b + 1], t0), a.total_q);
    const int s0 = min(max(a.cu_k[b], 0), a.total_k);
    const int s1 = min(max(a.cu_k[b + 1], s0), a.total_k);
    Nq = t1 - t0;
    Nkv = s1 - s0;
    if (MASK != 0) off = a.causal_br ? Nkv - Nq : 0;  // from the sequence's own lengths
    Nq = min(Nq, a.Nq);    // rows past the caller's max_seqlen_q bound are not computed
    if (q0 >= Nq) return;  // whole workgroup: block past this sequence's queries
    qbase = a.q + (int64_t)t0 * a.sqn + (int64_t)h * a.sqh;
    kbase = a.k + (int64_t)s0 * a.skn + (int64_t)kvh * a.skh;
    vbase = a.v + (int64_t)s0 * a.svn + (int64_t)kvh * a.svh;
    obase = a.o + (int64_t)t0 * a.son + (int64_t)h * a.soh;
    lbase = a.lse ? a.lse + (int64_t)h * a.total_q + t0 : nullptr;
    q_bytes = ((int64_t)(Nq - 1) * a.sqn + D) * 2;
  } else {
    qbase = a.q + (int64_t)b * a.sqb + (int64_t)h * a.sqh;
    kbase = a.k + (int64_t)b * a.skb + (int64_t)kvh * a.skh;
    vbase = a.v + (int64_t)b * a.svb + (int64_t)kvh * a.svh;
    obase = a.o + (int64_t)b * a.sob + (int64_t)h * a.soh;
    lbase = a.lse ? a.lse + ((int64_t)b * a.Hq + h) * a.Nq : nullptr;
  }

  // ---- Q fragment, register resident: B operand of S^T = K Q^T (rows >= Nq read as 0)
  u32x4 qf[KS];
  {
    const int64_t qblk = (int64_t)q0 * a.sqn;
    const auto rq = make_rsrc(qbase + qblk, clamp_bytes(q_bytes - 2 * qblk));
    const int32_t qoff = (32 * w + n) * (int32_t)a.sqn * 2 + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = bload16(rq, qoff + 32 * ks) ^ a.qsign;
  }

  // causal: query row i sees keys j <= i + off (off = 0 top-left, Nkv - Nq
  // bottom-right); keys past the block's last row + off are never visited.
  // band: row i sees i + off - WL <= j <= i + off + WR (an open side is a
  // bound no key reaches); tiles wholly left of the block's first row's band
  // or right of its last row's are never visited
  constexpr int kOpen = 1 << 30;
  const int WL = BAND ? (a.win_left < 0 ? kOpen : a.win_left) : 0;
  const int WR = BAND ? (a.win_right < 0 ? kOpen : a.win_right) : 0;
  const int kv_end = CAUSAL ? max(0, min(Nkv, q0 + kBM + off))
                            : (BAND ? max(0, min(Nkv, q0 + kBM + off + WR)) : Nkv);
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const int t_begin = BAND ? min(max(0, q0 + off - WL) / kBN, ntiles) : 0;
  // tiles every row of this block sees in full (no mask): below the block's
  // diagonal (band: and at or past its last row's lower bound) and before the
  // key tail
  const int n_full = CAUSAL ? max(0, min(q0 + off + 1, Nkv)) / kBN
                            : (BAND ? max(0, min(Nkv, q0 + off + WR + 1)) / kBN : Nkv / kBN);
  const int full_lo = BAND ? (max(0, q0 + kBM - 1 + off - WL) + kBN - 1) / kBN : 0;

  // ---- DMA geometry: wave w fills 1 KiB blocks NB*w .. NB*w+NB-1 of each
  //      K and V tile; lane l of block bk writes row RPB*bk + l/C, slot l%C,
  //      i.e. global chunk (l%C) ^ swz(row) of that row
  int32_t dk[NB], dv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int bk = NB * w + i;
    const int row = RPB * bk + lane / L::C;
    const int chunk = (lane % L::C) ^ swz<D>(row);
    dk[i] = row * (int32_t)a.skn * 2 + 16 * chunk;
    dv[i] = row * (int32_t)a.svn * 2 + 16 * chunk;
  }
  uint16_t* const ring = KVS == 1 ? smem : smem + grp * L::ELEMS;  // this key group's ring
  const uint32_t lds_k = lds_addr(ring + L::K0) + 1024 * NB * w;  // this wave's first block, stage 0
  const uint32_t lds_v = lds_addr(ring + L::V0) + 1024 * NB * w;
  auto dma_tile = [&](int t, int stage) {
    const int64_t ko = (int64_t)t * kBN * a.skn, vo = (int64_t)t * kBN * a.svn;
    // each load's range ends with the tile's last key row (none past Nkv)
    const int rows = min(Nkv - t * kBN, kBN);
    const i32x4 rk = rsrc_words(kbase + ko, rows > 0 ? ((rows - 1) * (int32_t)a.skn + D) * 2 : 0);
    const i32x4 rv = rsrc_words(vbase + vo, rows > 0 ? ((rows - 1) * (int32_t)a.svn + D) * 2 : 0);
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(rk, lds_k + 2 * stage * L::TILE + 1024 * i, dk[i]);
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(rv, lds_v + 2 * stage * L::TILE + 1024 * i, dv[i]);
  };

  // ---- LDS operand addresses (elements, relative to a 32-row subtile / 16-key chunk)
  // K operand of S^T: lane (n, hh) reads row n, chunk 2*ks + hh
  uint32_t ka[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    ka[ks] = opaque_lds(lds_addr(ring + L::K0) + 2 * (n * D + (((2 * ks + hh) ^ swz<D>(n)) << 3)));
  // V^T operand of P.V via transposed reads: lane (group g = lane/16, i = lane%16)
  // addresses row 8u + 4*(g/2) + i/4 of the 16-key chunk, head dims
  // 32*dt + 16*(g%2) + 4*(i%4) .. +3; read u = 0 / 1 give MFMA k-slots 0-3 / 4-7
  uint32_t va[DT][2];  // LDS byte addresses within stage 0's V tile
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 8 * u + 4 * (g >> 1) + (i >> 2);
        const int d = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
        va[dt][u] = opaque_lds(lds_addr(ring + L::V0) + 2 * (row * D + ((((d >> 3) ^ swz<D>(row)) << 3) | (d & 7))));
      }
  }

  // ---- online softmax state (fp32): reference max m (log2 domain), this
  //      lane's share of the running sum l, and the O^T accumulator
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;
  // bf16 only: this lane's share of the row sum of the P values as rounded for
  // the P.V MFMA (O is normalised by it; lse uses the fp32 sum l)
  float lt = 0.f;
  const float c = a.c;  // > 0
  const int wq_hi = q0 + 32 * w + 31 + off;  // last key any of this wave's rows sees
  const int wq_lo = q0 + 32 * w + off;       // band: this wave's first row's position

  // instruction order hints for the two MFMA phases of a tile (masks: 0x008
  // MFMA, 0x100 LDS read, 0x002 VALU): LDS reads run several MFMAs ahead of
  // their use, since a loaded LDS read takes some 250 cycles
  auto schedule_scores = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, kKLead, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto schedule_pv = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVLead, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu0, 0);
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValu1, 0);
    }
  };

  // mid() runs once per tile on every path, after the score MFMAs
  auto compute = [&](auto stage_tag, int t, auto masked_tag, auto&& mid) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int STG = decltype(stage_tag)::value;
    const int kb = t * kBN;
    bool act1 = true;
    if constexpr (MASKED) {
      if (kb >= Nkv || (CAUSAL && kb > wq_hi) || (BAND && (kb > wq_hi + WR || kb + kBN - 1 < wq_lo - WL))) {
        mid();
        return;
      }
      act1 = kb + 32 < Nkv && (!CAUSAL || kb + 32 <= wq_hi) && (!BAND || kb + 32 <= wq_hi + WR);
    }
    // S^T = K Q^T for the two 32-key subtiles; score register e of lane
    // (n, hh) is key 8*(e/4) + 4*hh + e%4 of its subtile
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    {
      constexpr uint32_t off0 = 2 * STG * L::TILE, off1 = off0 + 2 * 32 * D;
      if (act1) {
        // the two subtiles' MFMAs alternate, so the K reads (issued a few
        // MFMAs ahead) are consumed in the order they were issued
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s0 = mfma_32x32x16<BF16>(lds_load16(ka[ks] + off0), qf[ks], s0);
          s1 = mfma_32x32x16<BF16>(lds_load16(ka[ks] + off1), qf[ks], s1);
        }
        schedule_scores();
      } else {
        // (masked tiles only) the second subtile lies wholly outside this
        // wave's rows
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s0 = mfma_32x32x16<BF16>(lds_load16(ka[ks] + off0), qf[ks], s0);
      }
    }
    mid();

    if constexpr (MASKED) {
      // mask before the row max.  Score register e of this lane holds key
      // kb + 4 hh + c(e) of the first subtile, c(e) = 8 (e / 4) + e % 4 a
      // compile-time offset, and c(e) + 32 of the second; the key is visible
      // iff lo <= c <= hi for this lane's per-tile limits (64-bit, so open
      // band sides cannot overflow), a compare against an immediate per
      // register and no branches
      const int64_t base = (int64_t)kb + 4 * hh, pos = (int64_t)qrow + off;
      int64_t hi = (int64_t)Nkv - 1 - base;
      if (CAUSAL) hi = min(hi, pos - base);
      if (BAND) hi = min(hi, pos + WR - base);
      const int64_t lo = BAND ? pos - WL - base : 0;
      const int hi0 = (int)max(min(hi, (int64_t)64), (int64_t)-1);
      const int lo0 = (int)max(min(lo, (int64_t)64), (int64_t)0);
      const int hi1 = act1 ? hi0 - 32 : -1;
      const int lo1 = lo0 - 32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 8 * (e >> 2) + (e & 3);
        const bool vis0 = (c <= hi0) & (!BAND | (c >= lo0));
        const bool vis1 = (c <= hi1) & (!BAND | (c >= lo1));
        s0[e] = vis0 ? s0[e] : -INFINITY;
        s1[e] = vis1 ? s1[e] : -INFINITY;
      }
    }
    // P = exp2(s*c - m) against the current reference, its fp32 row sum and
    // the 16-bit B operand of P.V: pf[kk] holds keys 16*kk + 8u + 4*hh + t in
    // k-slot 4u + t
    u32x4 pf[4];
    float rs0, rs1;
    auto exps = [&](float mref) __attribute__((always_inline)) {
      rs0 = 0.f;
      rs1 = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s0[e], c, -mref));
        const float p1 = fast_exp2(__builtin_fmaf(s0[e + 1], c, -mref));
        const float p2 = fast_exp2(__builtin_fmaf(s1[e], c, -mref));
        const float p3 = fast_exp2(__builtin_fmaf(s1[e + 1], c, -mref));
        rs0 += p0 + p1;
        rs1 += p2 + p3;
        pf[e >> 3][(e & 7) >> 1] = pack2<BF16>(p0, p1);
        pf[2 + (e >> 3)][(e & 7) >> 1] = pack2<BF16>(p2, p3);
      }
    };
    // the reference moves only when some row has none yet (then P is not
    // formed against it), or when this lane's half row summed to more than
    // 2^10 on this tile (every P is then below 2^10 in the common path); the
    // row's max is formed only then
    bool move = __any(m == -INFINITY);
    if (!move) {
      exps(m);
      move = __any(rs0 + rs1 > kSumBound);
    }
    if (move) {
      float t3[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int j = 3 * i;
        const float x0 = j < 16 ? s0[j] : s1[j - 16];
        const float x1 = j + 1 < 16 ? s0[j + 1] : s1[j + 1 - 16];
        const float x2 = j + 2 < 16 ? s0[j + 2] : s1[j + 2 - 16];
        t3[i] = vmax(vmax(x0, x1), x2);
      }
      t3[10] = vmax(s1[14], s1[15]);
      const float u0 = vmax(vmax(t3[0], t3[1]), t3[2]), u1 = vmax(vmax(t3[3], t3[4]), t3[5]);
      const float u2 = vmax(vmax(t3[6], t3[7]), t3[8]), u3 = vmax(t3[9], t3[10]);
      const float mx = vmax(vmax(u0, u1), vmax(u2, u3));
      const float m_new = fmaxf(m, max_xor32(mx) * c);  // the row's max in the log2 domain
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      l *= alpha;
      if constexpr (BF16) lt *= alpha;
      m = m_new;
      exps(m == -INFINITY ? 0.f : m);  // rows with nothing visible yet get P = 0
    }
    l += rs0 + rs1;
    if constexpr (BF16) {
      // a bf16 P carries 8 significant bits and, under the lazy rescale, can
      // reach 2^10: normalising O by the sum of the rounded values makes O a
      // convex combination of V rows, so the rounding of a dominant P cancels
      // between O and its normaliser instead of scaling O by up to 2^-9
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) lt = sum2_bf16(pf[kk][j], lt);
    }

    // O^T += V^T P^T : A = V^T from transposed LDS reads, B = P^T from registers
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 2 || act1) {
        constexpr uint32_t base = 2 * STG * L::TILE;
        const uint32_t off = base + 2 * 16 * kk * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x2 lo = lds_read_tr16(va[dt][0] + off);
          const u32x2 hi = lds_read_tr16(va[dt][1] + off);
          oacc[dt] = mfma_32x32x16<BF16>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kk], oacc[dt]);
        }
      }
    }
    schedule_pv();
  };
  using full_t = std::false_type;
  using mask_t = std::true_type;
  using st0 = std::integral_constant<int, 0>;
  using st1 = std::integral_constant<int, 1>;
  using st2 = std::integral_constant<int, 2>;
  using st3 = std::integral_constant<int, 3>;

  // ---- this key group's tiles: first, first + KVS, ... below ntiles (every
  //      tile of [t_begin, ntiles) when KVS = 1)
  const int first = t_begin + grp;

  // ---- KV loop over a kStages-deep LDS ring filled by DMA: the loads of the
  //      group's tile kStages - 1 steps ahead are issued before tile t is
  //      computed, so every tile's loads have kStages - 1 tile computations to
  //      land.  After computing tile t a wave waits until only the loads of the
  //      group's tiles past its next one are outstanding (the next tile is in
  //      LDS), and the barrier publishes it to the workgroup; the stage
  //      refilled next was last read before that barrier (masked grids with
  //      one key group replace the barrier by the counted ring below).  Full
  //      tiles go in groups of kStages (stages 0 .. kStages-1); the rest
  //      (diagonal / key tail / band edges) take the masked path.
  constexpr int NDMA = 2 * NB;  // DMA instructions per wave per tile
  static_assert(kStages == 2 || (kStages - 2) * NDMA < 64, "vmcnt field");
  // s_waitcnt immediate for vmcnt <= vm (gfx9 encoding: vmcnt bits 3:0 and
  // 15:14, expcnt and lgkmcnt left at their maxima, i.e. unconstrained)
  constexpr int kVm1 = 0x0F70 | (NDMA & 15) | ((NDMA >> 4) << 14);
  constexpr int kVm2 = 0x0F70 | ((2 * NDMA) & 15) | (((2 * NDMA) >> 4) << 14);
  // wait until the group's tile after tt has landed: the tiles issued after
  // it are the group's tiles from tt + 2 KVS on, at most kStages - 2
  auto wait_next = [&](int tt) __attribute__((always_inline)) {
    const int ahead = min(kStages - 2, max(0, ntiles - tt - 2 * KVS + KVS - 1) / KVS);
    if (kStages == 4 && ahead >= 2)
      __builtin_amdgcn_s_waitcnt(kVm2);
    else if (ahead >= 1)
      __builtin_amdgcn_s_waitcnt(kVm1);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  // ---- counted ring (masked grids): per stage, the number of waves that
  //      have published their part of the stage's tile (`landed`) and the
  //      number done reading it (`read`), both counting up over the stage's
  //      reuses.  A wave starts its k-th tile once all waves have published
  //      it, publishes its own part of tile k+1 (its loads of it waited for)
  //      after tile k's scores, and after tile k refills the stage of tile
  //      k-1 with tile k+3 once all waves have read k-1.  A wave can thus run
  //      up to a tile ahead of the slowest: on diagonal and band-edge tiles
  //      the waves of a block have unequal work (subtiles above a wave's
  //      rows are skipped), and a barrier per tile made each of them cost
  //      its slowest wave.  Causal blocks keep the barrier protocol for their
  //      full tiles (where no wave has less work, and a barrier costs less
  //      than the counters) and count only on the diagonal ones; band blocks
  //      count on every tile.  Each wave tallies what all waves have added
  //      (exp_landed, exp_read); a tile right after a barrier needs no wait,
  //      and a full tile after counted ones takes a barrier first.  Every
  //      wait is bounded (a.ring_polls polls); one that runs out sets the
  //      block's failure word, and the block's output is written as NaN.
  const uint32_t landed = lds_addr(reinterpret_cast<const uint16_t*>(ring_cnt));
  const uint32_t read = landed + 16;
  const uint32_t failed = landed + 32;
  auto wait_count = [&](uint32_t addr, uint32_t target) __attribute__((always_inline)) {
    const int limit = a.ring_polls;
    int i = 0;
#pragma nounroll
    for (; i < limit; ++i) {
      uint32_t v;
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
      if (__builtin_amdgcn_readfirstlane(v) >= target) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (i == limit && lane == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(failed), "v"(1u) : "memory");
    asm volatile("" ::: "memory");  // no LDS access moves above the wait
  };
  // a wave's LDS instructions are served in issue order, so its reads of a
  // stage are done before its count of that stage goes up
  auto count_up = [&](uint32_t addr) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    if (lane == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(1u) : "memory");
  };
  // each wave's tally of what all waves have added to the counters, whether
  // the last step ended on a barrier, and whether it was counted
  uint32_t exp_landed[4] = {0, 0, 0, 0}, exp_read[4] = {0, 0, 0, 0};
  bool synced = true, prev_counted = false;
  auto step = [&](int tt, auto stage_tag, auto masked_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    if constexpr (kCounted && (MASKED || !CAUSAL)) {
      // a tile right after a barrier is in LDS for every wave already
      if (!synced) wait_count(landed + 4 * STG, exp_landed[STG]);
      compute(stage_tag, tt, masked_tag, [&]() __attribute__((always_inline)) {
        if (tt + 1 < ntiles) {
          if (tt + 2 < ntiles)
            __builtin_amdgcn_s_waitcnt(kVm1);
          else
            __builtin_amdgcn_s_waitcnt(0x0F70);
          count_up(landed + 4 * ((STG + 1) % 4));
          exp_landed[(STG + 1) % 4] += kWaves;
        }
      });
      count_up(read + 4 * STG);
      exp_read[STG] += kWaves;
      if (tt + 3 < ntiles) {
        // the stage of the previous tile: after a barrier every wave is done with it
        if (prev_counted) wait_count(read + 4 * ((STG + 3) % 4), exp_read[(STG + 3) % 4]);
        dma_tile(tt + 3, (STG + 3) % 4);
      }
      synced = false;
      prev_counted = true;
    } else if constexpr (kCounted) {
      // a full tile of a causal block: the barrier protocol, after a barrier
      // if the last step was counted
      if (!synced) barrier_nofence();
      if (tt + 3 < ntiles) dma_tile(tt + 3, (STG + 3) % 4);
      compute(stage_tag, tt, masked_tag, []() {});
      wait_next(tt);
      barrier_nofence();
      synced = true;
      prev_counted = false;
    } else {
      if (tt + KVS * (kStages - 1) < ntiles) dma_tile(tt + KVS * (kStages - 1), (STG + kStages - 1) % kStages);
      compute(stage_tag, tt, masked_tag, []() {});
      wait_next(tt);
      barrier_nofence();
    }
  };
  // the group's k-th tile sits in ring stage k % kStages
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (first + KVS * i < ntiles) dma_tile(first + KVS * i, i);
  wait_next(first - KVS);
  barrier_nofence();
  int t = first;
  auto masked_step = [&](int tt) __attribute__((always_inline)) {
    const int r = ((tt - first) / KVS) % kStages;
    if (r == 0)
      step(tt, st0{}, mask_t{});
    else if (r == 1)
      step(tt, st1{}, mask_t{});
    else if constexpr (kStages == 4) {
      if (r == 2)
        step(tt, st2{}, mask_t{});
      else
        step(tt, st3{}, mask_t{});
    }
  };
  if constexpr (BAND) {
    // band: the masked tiles left of the full ones, and as many more as put
    // the first full group in stage 0
    const int i_lo = (max(full_lo - first, 0) + KVS - 1) / KVS;
    const int f_start = first + KVS * kStages * ((i_lo + kStages - 1) / kStages);
    for (; t < f_start && t < ntiles; t += KVS) masked_step(t);
  }
  for (; t + KVS * (kStages - 1) < n_full; t += KVS * kStages) {
    step(t, st0{}, full_t{});
    step(t + KVS, st1{}, full_t{});
    if constexpr (kStages == 4) {
      step(t + 2 * KVS, st2{}, full_t{});
      step(t + 3 * KVS, st3{}, full_t{});
    }
  }
  for (; t < ntiles; t += KVS) masked_step(t);

  if constexpr (KVS >= 2) {
    // the groups with a tile fewer pass the barriers of the longest one's
    // last step
    const int span = max(ntiles - t_begin, 0);
    const int count = (max(span - grp, 0) + KVS - 1) / KVS;  // this group's tiles
    for (int j = count; j < (span + KVS - 1) / KVS; ++j) barrier_nofence();
    // ---- merge: groups 1 .. KVS-1 leave (m, l, O^T) in LDS (the rings are
    //      free: every LDS read and load of every ring completed before the
    //      last barrier), group 0 takes them up with the rescale identity
    //      O = sum_g 2^(m_g - M) O_g, l likewise, M = max_g m_g
    constexpr int NC = 1 + 4 * DT;  // 16-byte chunks per lane: (m, l), then O^T
    static_assert((KVS - 1) * RW * NC * 64 * 16 <= KVS * L::ELEMS * 2, "the exchange fits in the rings");
    f32x4* const xch = reinterpret_cast<f32x4*>(smem) + (w * NC) * 64 + lane;
    constexpr int XG = RW * NC * 64;  // f32x4 entries per group's exchange region
    if (grp != 0) {
      f32x4* const x = xch + (grp - 1) * XG;
      x[0] = f32x4{m, l, lt, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          x[(1 + 4 * dt + c4) * 64] =
              f32x4{oacc[dt][4 * c4], oacc[dt][4 * c4 + 1], oacc[dt][4 * c4 + 2], oacc[dt][4 * c4 + 3]};
    }
    __syncthreads();
    if (grp != 0) return;
#pragma unroll
    for (int g = 1; g < KVS; ++g) {
      const f32x4* const x = xch + (g - 1) * XG;
      const f32x4 ml = x[0];
      const float mx = fmaxf(m, ml[0]);
      const float mu = (mx == -INFINITY) ? 0.f : mx;
      const float a0 = fast_exp2(m - mu), a1 = fast_exp2(ml[0] - mu);
      l = a0 * l + a1 * ml[1];
      if constexpr (BF16) lt = a0 * lt + a1 * ml[2];
      m = mx;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4 o1 = x[(1 + 4 * dt + c4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[dt][4 * c4 + e] = a0 * oacc[dt][4 * c4 + e] + a1 * o1[e];
        }
    }
  }

  // ---- epilogue: O = O^T / l, cast, store; lse = (m + log2 l) ln 2
  l = sum_xor32(l);
  const float ln = BF16 ? sum_xor32(lt) : l;  // O's normaliser
  // The lane's row and half are re-derived from the lane counter here rather
  // than kept live across the KV loop (which would cost two spilled registers).
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int hh_e = lane_e >> 5;
  const int qrow_e = q0 + 32 * w + (lane_e & 31);
  // a counted ring whose wait ran out: the block's output is not to be trusted
  bool lost = false;
  if constexpr (kCounted) {
    uint32_t f;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(f) : "v"(failed) : "memory");
    lost = __builtin_amdgcn_readfirstlane(f) != 0;
  }
  // O goes through LDS so that the stores cover whole rows: the wave's own
  // slice of the ring once every wave is done with it (one key group), or
  // its merge slot (several)
  const float inv = lost ? __builtin_nanf("") : (ln > 0.f) ? 1.f / ln : 0.f;
  if constexpr (kCounted) barrier_nofence();  // the ring: every wave past its last tile
  const uint32_t stg = lds_addr(smem) + (KVS == 1 ? w * 32 * 2 * D : w * (1 + 4 * DT) * 1024);
  static_assert(KVS > 1 || kWaves * 32 * 2 * D <= L::ELEMS * 2, "every wave's rows fit in the ring");
  static_assert(KVS == 1 || (1 + 4 * DT) * 1024 >= 32 * 2 * D, "a wave's rows fit in its merge slot");
  store_tile_rows<D, BF16>(stg, oacc, inv, obase, a.son, q0 + 32 * w, Nq);
  if (qrow_e < Nq && lbase != nullptr && hh_e == 0)
    lbase[qrow_e] = lost ? __builtin_nanf("") : (l > 0.f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// 128-row blocks: dense grids too small for 256-row blocks take two key groups
// (8 waves); packed batches of short sequences take one (4 waves, two
// workgroups per CU, so one block's start and end overlap the other's loop)
template <int D, bool BF16, int MASK, bool VARLEN>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  if (a.rows == 128) {
    if constexpr (VARLEN)
      hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, MASK, VARLEN, 4, 1>), dim3(a.nblocks), dim3(64 * 4), 0, stream,
                         a);
    else if constexpr (D == 64)
      hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, MASK, VARLEN, 4, 3>), dim3(a.nblocks), dim3(64 * 12), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, MASK, VARLEN, 4, 2>), dim3(a.nblocks), dim3(64 * 8), 0, stream,
                         a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, MASK, VARLEN, 8, 1>), dim3(a.nblocks), dim3(64 * 8), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool VARLEN>
hipError_t launch_c(const FwdArgs& a, int mask, hipStream_t stream) {
  if (mask == 2) return launch_t<D, BF16, 2, VARLEN>(a, stream);
  return mask == 1 ? launch_t<D, BF16, 1, VARLEN>(a, stream) : launch_t<D, BF16, 0, VARLEN>(a, stream);
}

template <int D, bool VARLEN>
hipError_t launch_d(const FwdArgs& a, bool bf16, int mask, hipStream_t stream) {
  return bf16 ? launch_c<D, true, VARLEN>(a, mask, stream) : launch_c<D, false, VARLEN>(a, mask, stream);
}

template <bool VARLEN>
hipError_t launch_v(const FwdArgs& a, int D, bool bf16, int mask, hipStream_t stream) {
  if (D == 64) return launch_d<64, VARLEN>(a, bf16, mask, stream);
  return launch_d<128, VARLEN>(a, bf16, mask, stream);
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, int mask, bool varlen, hipStream_t stream) {
  return varlen ? launch_v<true>(a, D, bf16, mask, stream) : launch_v<false>(a, D, bf16, mask, stream);
}

}  // namespace attn
