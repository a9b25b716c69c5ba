// KV-cache decode attention and the cache writer for gfx950.
//
// What it computes: for every (batch, q head), o = softmax(scale * q K^T) V over
// cache slots [0, cache_len) and lse -- the decode kernel of the
// "Triton-FlashAttention" README (decode phase): one new query token, every
// cached slot visible, cache_len a runtime value, GQA indexing as in prefill.
// The online-softmax recurrence and its rescale identity are those of "Skill:
// Write a Triton Attention Kernel" (Required reasoning process, step 5) and
// "FlashAttention Kernel Optimization" (Online Softmax).
//
// gfx950 design (the page's kernel uses one program per (batch, head); this
// one is split along the cache so that a 16-unit problem fills 256 CUs):
//   * a workgroup = 4 wave64s handles one (batch, kv head), up to 16 of the q
//     heads that share it (K/V are read from HBM once for the whole group), and
//     one contiguous chunk ("split") of the cache, normally a single 128-key
//     tile, so that all of a workgroup's loads are in flight at once and up to
//     four workgroups share a CU.
//   * each wave takes 32 keys of a tile.  K goes straight from HBM into
//     registers in MFMA operand layout (buffer loads; keys past the split end
//     read as zero and are masked); V is staged through LDS transposed, the
//     layout the P.V MFMA needs.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32; the q heads of the
//     group are the 16 MFMA columns.  K rows are fed in a permuted order so the
//     score registers are directly the B operand of the P.V MFMA.
//   * each workgroup merges its 4 waves' (m, l, o) in LDS.  With one split it
//     writes the normalised output; otherwise it stores its partial
//     (m, l, unnormalised o) and a second, small kernel merges the partials of
//     every (batch, q head) with the same max/rescale identity, in parallel
//     over head-dim columns and split groups.  The kernel boundary orders the
//     two, so no workgroup waits on or signals another.  (A single kernel in
//     which the last workgroup to finish merges measured slower on MI355X:
//     device-coherent publication costs every workgroup a store drain and an
//     atomic, more than the second launch costs.)
#include <atomic>
#include <mutex>

#include "attn.h"
#include "kernel_common.hpp"
#include "launch.hpp"

namespace attn {

namespace {

constexpr int kDT = 128;        // keys per tile (32 per wave)
constexpr int kDecodeWgsPerCu = 2;  // workgroups per CU the register budget is sized for
constexpr int kMaxSplits = 64;  // partials merged by one combine (the host keeps nsplit <= this)
constexpr int kPartPad = 4;     // per-head partial: m, l, 2 pad, o[D] -> 16-byte aligned o

// MODE 0: one length for every sequence; 1: per-sequence lengths; 2: per-sequence
// lengths over a paged cache.  WINDOW: a sliding window hides the slots before
// len - 1 - window_left (without it none of that code is compiled in)
template <int D, bool BF16, int MODE, bool WINDOW>
__global__ __launch_bounds__(256, kDecodeWgsPerCu) void decode_kernel(const DecodeArgs a) {
  constexpr bool VARLEN = MODE >= 1;
  constexpr bool PAGED = MODE == 2;
  constexpr int KS = D / 32;                 // k-steps of the score MFMA
  constexpr int NDT = D / 16;                // 16-wide head-dim tiles of O
  constexpr int VLD = kDT;                   // V^T row pitch (elements); 16-byte groups XOR-swizzled
  constexpr int VBLK = (kDT / 4) * (D / 8);  // 4x8 V blocks per tile
  constexpr int VPT = VBLK / 256;            // V blocks per thread
  static_assert(VBLK % 256 == 0, "V blocks divide evenly");
  constexpr int RED_FLOATS = 128 + 4 * 16 * (D + 4);  // wave merge: m[4][16], l[4][16], o[4][16][D + 4]
  constexpr int LDS_BYTES = (RED_FLOATS * 4 > D * VLD * 2) ? RED_FLOATS * 4 : D * VLD * 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];  // V^T stage, then the merges
  uint16_t* const vt = reinterpret_cast<uint16_t*>(lds);

  // Consecutive workgroups are dealt round-robin to the XCDs.  With one length
  // for every sequence the chunk index runs fastest (each (batch, kv head)
  // spread over all XCDs).  With per-sequence lengths the (batch, kv head)
  // index runs fastest: all kv heads of a sequence share its length, so the
  // chunks that cover short sequences spread over every XCD instead of piling
  // onto the XCDs that chunks 0, 1, ... would map to.
  const int unit = a.unit_fast ? blockIdx.x : blockIdx.z;
  const int hgi = blockIdx.y;
  const int split = a.unit_fast ? blockIdx.z : blockIdx.x;
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int h0 = kvh * a.group + hgi * a.heads_per_wg;  // first q head of this workgroup
  const int nh = min(a.heads_per_wg, a.group - hgi * a.heads_per_wg);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane & 15;  // MFMA column = q head within the group
  const int rg = lane >> 4;   // 4-row group of the MFMA output / k-group of operands

  // this sequence's length (VARLEN: per-sequence lengths clamped to [0,
  // cache_len]).  A chunk wholly past it has nothing to do: with several chunks
  // the combine merges only the chunks that cover the sequence, so it writes
  // nothing; a single chunk (length 0) still writes o = 0 and lse = -inf below.
  // Without per-sequence lengths every chunk is non-empty and none of this is
  // compiled in (the test would delay the first loads).
  const int seq_len = VARLEN ? min(max(a.lens[b], 0), a.cache_len) : a.cache_len;
  // sliding window: slots below kvis are hidden and never read; chunks start
  // at the tile that holds kvis
  const int kvis = WINDOW ? max(0, seq_len - 1 - a.window_left) : 0;
  const int k0 = (kvis & ~(kDT - 1)) + split * a.rows_per_split;
  const int k1 = min(seq_len, k0 + a.rows_per_split);
  if (VARLEN && a.nsplit > 1 && k0 >= seq_len) return;  // uniform over the workgroup

  // q heads as the B operand.  Columns beyond nh repeat the group's last head:
  // MFMA columns never mix, and those columns' results are never stored.  (A
  // load predicated on col < nh makes the compiler wait for it before issuing
  // anything else, costing every workgroup one memory latency.)
  u32x4 qf[KS];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.sqb + (int64_t)(h0 + min(col, nh - 1)) * a.sqh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = load16(qp + 32 * ks + 8 * rg) ^ a.qsign;
  }

  const uint16_t* kbase = a.k + (PAGED ? 0 : (int64_t)b * a.skb) + (int64_t)kvh * a.skh;
  const uint16_t* vbase = a.v + (PAGED ? 0 : (int64_t)b * a.svb) + (int64_t)kvh * a.svh;
  // MFMA row i of key group gi reads key 8*(i/4) + 4*gi + i%4 of the wave's 32,
  // so that lane (col, rg) holds keys 8*rg .. 8*rg+7 in its score registers.
  const int krow = 32 * w + 8 * (col >> 2) + (col & 3);
  const int32_t koff = krow * (int32_t)a.skn * 2 + 16 * rg;
  // V blocks of 4 keys x 8 columns.  With the swizzled layout, 16 consecutive
  // lanes cover one 256-byte row per load and V^T group g of row d sits at
  // 16-byte slot g ^ vswz(d), which keeps both the transposing writes and the
  // MFMA operand reads free of LDS bank conflicts without padding.
  int32_t voff[VPT][4];
  int vkvg[VPT], vdc[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int id = tid + 256 * j;
    vdc[j] = id % (D / 8);
    vkvg[j] = id / (D / 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) voff[j][r] = (4 * vkvg[j] + r) * (int32_t)a.svn * 2 + 16 * vdc[j];
  }
  auto vt_at = [&](int d, int key) {  // element offset of V^T[d][key], key a multiple of 4
    const int sw = (d ^ (d >> 3)) & 15;
    return d * VLD + 8 * ((key >> 3) ^ sw) + (key & 7);
  };

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{};
  float m = -INFINITY;  // running max of this lane's head column (log2 domain)
  float l = 0.f;        // this lane's share of the running sum
  const float c = a.c;

  // one tile's loads: K straight into MFMA operand registers, V into registers
  // for the transposed LDS write; keys >= k1 read as zero
  struct Tile {
    u32x4 kf[2][KS];
    u32x4 v[VPT][4];
  };
  auto load_tile = [&](Tile& T, int kb) {
    if constexpr (PAGED) {
      // Slot r lives in page block_table[b][r >> lg_ps], row r & (page size - 1).
      // Rows past the chunk re-read its last row and rows before the window
      // its first visible one (their scores are masked, their P is 0), so no
      // load is predicated and no hidden slot or its page is touched.  A
      // wave's 32 K rows and a (wave, j) group of V rows span at most two pages
      // (page size >= 16, groups aligned): their page ids are uniform loads.
      const int last = k1 - 1;
      auto row = [&](int r) __attribute__((always_inline)) { return min(WINDOW ? max(r, kvis) : r, last); };
      const int wu = __builtin_amdgcn_readfirstlane(w);
      const int32_t* tb = a.block_table + (int64_t)b * a.mbps;
      const int rmask = (1 << a.lg_ps) - 1;
      auto page = [&](int r) __attribute__((always_inline)) {
        return (int64_t)min(max(tb[r >> a.lg_ps], 0), a.num_pages - 1);
      };
      const int kw0 = kb + 32 * wu;
      const int64_t kp_lo = page(row(kw0)), kp_hi = page(row(kw0 + 16));
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int rr = row(kb + krow + 4 * gi);
        const int64_t pg = rr >= kw0 + 16 ? kp_hi : kp_lo;
        const uint16_t* kp = kbase + pg * a.skb + (int64_t)(rr & rmask) * a.skn + 8 * rg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) T.kf[gi][ks] = load16_nt(kp + 32 * ks);
      }
      constexpr int VROWS = 2048 / D;  // V rows one wave loads per j
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int vs = kb + VROWS * (wu + 4 * j);
        const int64_t vp_lo = page(row(vs)), vp_hi = page(row(vs + 16));
        const int g0 = kb + 4 * vkvg[j];
        const uint16_t* vb = vbase + (g0 >= vs + 16 ? vp_hi : vp_lo) * a.svb + 8 * vdc[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) T.v[j][r] = load16_nt(vb + (int64_t)(row(g0 + r) & rmask) * a.svn);
      }
      return;
    }
    const int64_t ko = (int64_t)kb * a.skn, vo = (int64_t)kb * a.svn;
    // keys of this split in the tile: each load's range ends with the last
    // one (the tile's loads read its rows 0 .. kDT - 1 only)
    const int rows = min(k1 - kb, kDT);
    const auto rk = make_rsrc(kbase + ko, rows > 0 ? ((rows - 1) * (int32_t)a.skn + D) * 2 : 0);
    const auto rv = make_rsrc(vbase + vo, rows > 0 ? ((rows - 1) * (int32_t)a.svn + D) * 2 : 0);
    if (WINDOW && kb < kvis) {
      // the window's lead-in tile: rows before kvis re-read row kvis (their
      // scores are masked, their P is 0), so hidden slots are never read
      const int f = kvis - kb;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          T.kf[gi][ks] = bload16_nt(rk, max(krow + 4 * gi, f) * (int32_t)a.skn * 2 + 16 * rg + 64 * ks);
#pragma unroll
      for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          T.v[j][r] = bload16_nt(rv, max(4 * vkvg[j] + r, f) * (int32_t)a.svn * 2 + 16 * vdc[j]);
      return;
    }
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.kf[gi][ks] = bload16_nt(rk, koff + gi * 4 * (int32_t)a.skn * 2 + 64 * ks);
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) T.v[j][r] = bload16_nt(rv, voff[j][r]);
  };
  auto compute_tile = [&](const Tile& T, int kb, bool first) {
    if (!first) __syncthreads();  // the previous tile's V^T reads are done
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 lo{halves<0x05040100u>(T.v[j][0][q], T.v[j][1][q]), halves<0x05040100u>(T.v[j][2][q], T.v[j][3][q])};
        const u32x2 hi{halves<0x07060302u>(T.v[j][0][q], T.v[j][1][q]), halves<0x07060302u>(T.v[j][2][q], T.v[j][3][q])};
        *reinterpret_cast<u32x2*>(vt + vt_at(8 * vdc[j] + 2 * q, 4 * vkvg[j])) = lo;
        *reinterpret_cast<u32x2*>(vt + vt_at(8 * vdc[j] + 2 * q + 1, 4 * vkvg[j])) = hi;
      }
    }
    __syncthreads();
    const int kw0 = kb + 32 * w;  // first key of this wave
    if (kw0 >= k1 || (WINDOW && kw0 + 32 <= kvis)) return;  // no key of this wave in range
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma_16x16x32<BF16>(T.kf[0][ks], qf[ks], s0);
      s1 = mfma_16x16x32<BF16>(T.kf[1][ks], qf[ks], s1);
    }
    // lane (col, rg): s0[e] is key kw0 + 8*rg + e, s1[e] is key kw0 + 8*rg + 4 + e
    if (WINDOW && kw0 < kvis) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kw0 + 8 * rg + e;
        s0[e] = (key >= kvis) ? s0[e] : -INFINITY;
        s1[e] = (key + 4 >= kvis) ? s1[e] : -INFINITY;
      }
    }
    if (kw0 + 32 > k1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kw0 + 8 * rg + e;
        s0[e] = (key < k1) ? s0[e] : -INFINITY;
        s1[e] = (key + 4 < k1) ? s1[e] : -INFINITY;
      }
    }
    float mx = vmax(vmax(vmax(s0[0], s0[1]), vmax(s0[2], s0[3])), vmax(vmax(s1[0], s1[1]), vmax(s1[2], s1[3])));
    mx = max_xor32(max_xor16(mx)) * c;
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = fast_exp2(__builtin_fmaf(s0[e], c, -m_use));
      p[4 + e] = fast_exp2(__builtin_fmaf(s1[e], c, -m_use));
    }
    l = l * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
    m = m_new;
    const u32x4 pf{pack2<BF16>(p[0], p[1]), pack2<BF16>(p[2], p[3]), pack2<BF16>(p[4], p[5]),
                   pack2<BF16>(p[6], p[7])};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      oacc[dt] *= alpha;
      oacc[dt] = mfma_16x16x32<BF16>(load16(vt + vt_at(16 * dt + col, 32 * w + 8 * rg)), pf, oacc[dt]);
    }
  };

  // tiles of this split, the next tile's loads always issued before the
  // current tile is consumed (two tiles in flight per workgroup)
  Tile ta, tb;
  if (!PAGED || k0 < k1) load_tile(ta, k0);  // (an empty chunk has no row to look up)
  for (int kb = k0; kb < k1; kb += 2 * kDT) {
    const bool has_b = kb + kDT < k1;
    if (has_b) load_tile(tb, kb + kDT);
    compute_tile(ta, kb, kb == k0);
    if (!has_b) break;
    if (kb + 2 * kDT < k1) load_tile(ta, kb + 2 * kDT);
    compute_tile(tb, kb + kDT, false);
  }
  __syncthreads();  // V^T reads done: the LDS is reused for the merges below

  // ---- merge the 4 waves in LDS: per wave m[16], l[16] and the o rows of the
  //      group's nh heads (fp32), rows padded to D + 4 floats so that the
  //      heads of a wave start on different banks
  float* red = reinterpret_cast<float*>(lds);
  float* rm = red;       // [4][16]
  float* rl = red + 64;  // [4][16]
  constexpr int RP = D + 4;  // padded row of o: heads of one wave start on different banks
  float* ro = red + 128; // [4][16][RP]
  l = sum_xor32(sum_xor16(l));
  if (rg == 0) {
    rm[w * 16 + col] = m;
    rl[w * 16 + col] = l;
  }
  if (col < nh) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<f32x4*>(ro + (w * 16 + col) * RP + 16 * dt + 4 * rg) = oacc[dt];
  }
  __syncthreads();

  // thread -> (head hn, SL-wide slice of the head dim)
  constexpr int SL = D / 16;
  const int hn = tid >> 4;
  const int d0 = (tid & 15) * SL;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, rm[ww * 16 + hn]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float Ls = 0.f;
  float acc[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const float sc = fast_exp2(rm[ww * 16 + hn] - Mu);
    Ls += sc * rl[ww * 16 + hn];
#pragma unroll
    for (int j = 0; j < SL; ++j) acc[j] += sc * ro[(ww * 16 + hn) * RP + d0 + j];
  }

  auto store_lse = [&](int head, float Mx, float Lx) {
    if (a.lse != nullptr) a.lse[(int64_t)b * a.Hq + h0 + head] = (Lx > 0.f) ? (Mx + __log2f(Lx)) * kLn2 : -INFINITY;
  };

  if (a.nsplit == 1) {
    if (hn < nh) {
      const float inv = (Ls > 0.f) ? 1.f / Ls : 0.f;
      uint16_t* op = a.o + (int64_t)b * a.sob + (int64_t)(h0 + hn) * a.soh + d0;
      if constexpr (SL == 8) {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack2<BF16>(acc[2 * j] * inv, acc[2 * j + 1] * inv);
        store16(op, v);
      } else {
        static_assert(SL == 4, "D is 64 or 128");
        *reinterpret_cast<u32x2*>(op) = u32x2{pack2<BF16>(acc[0] * inv, acc[1] * inv), pack2<BF16>(acc[2] * inv, acc[3] * inv)};
      }
      if ((tid & 15) == 0) store_lse(hn, M, Ls);
    }
    return;
  }

  // ---- several splits: publish this split's partial (m, l, o[D]); a second
  //      kernel merges them (the kernel boundary orders the two)
  constexpr int HP = D + kPartPad;  // floats per head in a partial
  if (hn < nh) {
    const int64_t slot = (int64_t)unit * a.hgroups + hgi;
    float* pr = a.part + ((slot * a.max_splits + split) * a.heads_per_wg + hn) * HP;
    if ((tid & 15) == 0) *reinterpret_cast<f32x4*>(pr) = f32x4{M, Ls, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < SL; j += 4)
      *reinterpret_cast<f32x4*>(pr + kPartPad + d0 + j) = f32x4{acc[j], acc[j + 1], acc[j + 2], acc[j + 3]};
  }
}

// Merge the split partials of one (batch, q head): o = sum_s e^(m_s - M) o_s /
// sum_s e^(m_s - M) l_s and lse = M + ln(sum_s e^(m_s - M) l_s) (log2 domain
// inside).  Thread -> (4-wide column of o, group of splits strided by G); all
// of a thread's loads (its splits' o columns and m, and the (m, l) of split
// `lane`) are issued first.  Lane s of every wave holds split s's (m, l), so M
// and the denominator come from wave reductions, with no serial loop over the
// splits.  One barrier: the column sums across the split groups of the 4 waves.
template <int D, bool BF16, bool VARLEN>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeArgs a) {
  constexpr int HP = D + kPartPad;
  constexpr int C4 = D / 4;    // 4-wide columns
  constexpr int G = 256 / C4;  // split groups
  constexpr int PER = (kMaxSplits + G - 1) / G;  // splits per thread at most
  static_assert(kMaxSplits <= 64 && G * PER <= 64, "one lane per split holds its (m, l)");
  __shared__ __attribute__((aligned(16))) float sacc[G * D];
  const int unit = a.unit_fast ? blockIdx.x : blockIdx.z;  // batch x kv head
  const int hgi = blockIdx.y;
  const int hx = a.unit_fast ? blockIdx.z : blockIdx.x;  // head within the group
  const int nh = min(a.heads_per_wg, a.group - hgi * a.heads_per_wg);
  if (hx >= nh) return;  // whole workgroup: uniform
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int h = kvh * a.group + hgi * a.heads_per_wg + hx;
  // chunks that cover this sequence (all of them without per-sequence lengths)
  int ns = a.nsplit;
  if (VARLEN) {
    const int seq_len = min(max(a.lens[b], 0), a.cache_len);
    const int kbeg = (a.window_left >= 0 ? max(0, seq_len - 1 - a.window_left) : 0) & ~(kDT - 1);
    ns = min(ns, (seq_len - kbeg + a.rows_per_split - 1) / a.rows_per_split);
  }
  const int64_t slot = (int64_t)unit * a.hgroups + hgi;
  const float* base = a.part + (slot * a.max_splits * a.heads_per_wg + hx) * HP;
  const int64_t sstride = (int64_t)a.heads_per_wg * HP;  // between splits
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int dq = tid % C4, sg = tid / C4;
  f32x4 ov[PER];
  float mi[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = sg + i * G;
    ov[i] = (s < ns) ? *reinterpret_cast<const f32x4*>(base + s * sstride + kPartPad + 4 * dq) : f32x4{};
    mi[i] = (s < ns) ? base[s * sstride] : -INFINITY;
  }
  float ms = -INFINITY, ls = 0.f;
  if (lane < ns) {
    const f32x4 ml = *reinterpret_cast<const f32x4*>(base + lane * sstride);
    ms = ml[0];
    ls = ml[1];
  }
  const float M = wave_max(ms);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float L = wave_sum((lane < ns) ? fast_exp2(ms - Mu) * ls : 0.f);
  f32x4 o4 = f32x4{};
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sg + i * G < ns) o4 += fast_exp2(mi[i] - Mu) * ov[i];
  *reinterpret_cast<f32x4*>(sacc + 4 * (sg * C4 + dq)) = o4;
  __syncthreads();
  if (tid < C4) {
    f32x4 t = f32x4{};
#pragma unroll
    for (int g = 0; g < G; ++g) t += *reinterpret_cast<const f32x4*>(sacc + 4 * (g * C4 + tid));
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    uint16_t* op = a.o + (int64_t)b * a.sob + (int64_t)h * a.soh + 4 * tid;
    *reinterpret_cast<u32x2*>(op) = u32x2{pack2<BF16>(t[0] * inv, t[1] * inv), pack2<BF16>(t[2] * inv, t[3] * inv)};
    if (tid == 0 && a.lse != nullptr) a.lse[(int64_t)b * a.Hq + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
}

template <int D, bool BF16, int MODE>
hipError_t launch_v(const DecodeArgs& a, int B, hipStream_t stream) {
  const unsigned units = (unsigned)(B * a.Hkv);
  const dim3 g1 = a.unit_fast ? dim3(units, a.hgroups, a.nsplit) : dim3(a.nsplit, a.hgroups, units);
  if (a.window_left >= 0)
    hipLaunchKernelGGL((decode_kernel<D, BF16, MODE, true>), g1, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, BF16, MODE, false>), g1, dim3(256), 0, stream, a);
  if (a.nsplit > 1) {
    const dim3 g2 = a.unit_fast ? dim3(units, a.hgroups, a.heads_per_wg) : dim3(a.heads_per_wg, a.hgroups, units);
    hipLaunchKernelGGL((decode_combine_kernel<D, BF16, (MODE >= 1)>), g2, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_t(const DecodeArgs& a, int B, hipStream_t stream) {
  if (a.block_table) return launch_v<D, BF16, 2>(a, B, stream);
  return a.lens ? launch_v<D, BF16, 1>(a, B, stream) : launch_v<D, BF16, 0>(a, B, stream);
}

// ---- cache writer: a plain 16-byte-vector copy of T rows per (batch, kv head)
__global__ __launch_bounds__(256) void cache_write_kernel(const CacheWriteArgs a) {
  const int cpr = a.D / 8;  // 16-byte chunks per row
  const int64_t total = a.rows * cpr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool isv = i >= total;
    const int64_t j = isv ? i - total : i;
    const int c8 = (int)(j % cpr);
    const int64_t r = j / cpr;
    const int t = (int)(r % a.T);
    const int64_t bh = r / a.T;
    const int kvh = (int)(bh % a.Hkv);
    const int64_t b = bh / a.Hkv;
    if (!isv) {
      const u32x4 x = load16(a.kn + b * a.sknb + kvh * a.sknh + t * a.sknn + 8 * c8);
      store16(a.kc + b * a.skcb + kvh * a.skch + (int64_t)(a.pos + t) * a.skcn + 8 * c8, x);
    } else {
      const u32x4 x = load16(a.vn + b * a.svnb + kvh * a.svnh + t * a.svnn + 8 * c8);
      store16(a.vc + b * a.svcb + kvh * a.svch + (int64_t)(a.pos + t) * a.svcn + 8 * c8, x);
    }
  }
}

// ---- paged cache writer: row t of sequence b goes to slot pos[b] + t, i.e. row
//      (pos[b] + t) & (page size - 1) of page block_table[b][(pos[b] + t) >> lg_ps].
//      Slots outside [0, mbps * page size) are skipped; page ids are clamped
//      into the pool.
__global__ __launch_bounds__(256) void cache_write_paged_kernel(const CacheWritePagedArgs a) {
  const int cpr = a.D / 8;  // 16-byte chunks per row
  const int64_t total = a.rows * cpr;
  const int64_t cap = (int64_t)a.mbps << a.lg_ps;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool isv = i >= total;
    const int64_t j = isv ? i - total : i;
    const int c8 = (int)(j % cpr);
    const int64_t r = j / cpr;
    const int t = (int)(r % a.T);
    const int64_t bh = r / a.T;
    const int kvh = (int)(bh % a.Hkv);
    const int b = (int)(bh / a.Hkv);
    const int64_t slot = (int64_t)a.pos[b] + t;
    if (slot < 0 || slot >= cap) continue;
    const int64_t pg = min(max(a.block_table[(int64_t)b * a.mbps + (slot >> a.lg_ps)], 0), a.num_pages - 1);
    const int64_t row = slot & ((1 << a.lg_ps) - 1);
    if (!isv) {
      const u32x4 x = load16(a.kn + b * a.sknb + kvh * a.sknh + t * a.sknn + 8 * c8);
      store16(a.kp + pg * a.skpp + kvh * a.skph + row * a.skpn + 8 * c8, x);
    } else {
      const u32x4 x = load16(a.vn + b * a.svnb + kvh * a.svnh + t * a.svnn + 8 * c8);
      store16(a.vp + pg * a.svpp + kvh * a.svph + row * a.svpn + 8 * c8, x);
    }
  }
}

// ---- the split partials of attn_decode_noalloc, for callers that cannot
//      allocate: a fixed array in the library's own device memory, one copy
//      per GPU, held until the process ends.  Every such call on a GPU uses
//      that GPU's copy (calls that overlap on one GPU race on it).  Each call
//      writes every partial its combine reads, so nothing needs clearing.
static __device__ __align__(256) uint8_t scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;  // devices whose scratch address is remembered
std::atomic<void*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t decode_scratch_address(hipStream_t stream, void** addr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      // the symbol's address on `dev`, looked up with `dev` current (each GPU
      // holds its own copy of the array at its own address); host code uses
      // only this address, never the array's name
      int cur = 0;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess) return e;
      if (e2 != hipSuccess) return e2;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}

hipError_t launch_cache_write_paged(const CacheWritePagedArgs& a, hipStream_t stream) {
  const int64_t work = 2 * a.rows * (a.D / 8);
  const int64_t blocks = (work + 255) / 256;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(cache_write_paged_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int B, int D, bool bf16, hipStream_t stream) {
  if (D == 64) return bf16 ? launch_t<64, true>(a, B, stream) : launch_t<64, false>(a, B, stream);
  return bf16 ? launch_t<128, true>(a, B, stream) : launch_t<128, false>(a, B, stream);
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  const int64_t work = 2 * a.rows * (a.D / 8);
  const int64_t blocks = (work + 255) / 256;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(cache_write_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
