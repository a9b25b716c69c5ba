// Fused attention forward (prefill) for gfx950.
//
// What it computes: O = softmax(scale * Q K^T + mask) V and lse, following the
// tiled online-softmax method of "Skill: Write a Triton Attention Kernel"
// (Required reasoning process, steps 1-9) and "FlashAttention Kernel
// Optimization" (Online Softmax; Tiled Computation; Causal Masking), with GQA
// head sharing as in the "Triton-FlashAttention" README (GQA phase).
//
// gfx950 design (not the pages' Triton tiling):
//   * one workgroup = 4 wave64s = 128 query rows of one q head; each wave owns
//     32 rows for the whole KV loop.  Two workgroups share a CU.
//   * KV tiles of 64 rows are staged in LDS, double buffered: K row-major, V
//     transposed (head-dim major) so both MFMA operands are single 16-byte LDS
//     reads.  Global loads for tile t+1 are issued before tile t is computed;
//     they are buffer loads whose hardware range check returns zeros past the
//     last key, so ragged tails need no branches.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//     Q is the register-resident B operand and each lane ends up owning one
//     query row's scores.  The K rows fed to the MFMA are permuted (bits 2 and
//     3 of the row index swapped) so that the fp32 score registers of a lane
//     are exactly the B operand layout of the P.V MFMA: no data movement
//     between the two contractions.
//   * online softmax in the log2 domain: t = s * scale * log2(e); the row max
//     needs one cross-lane exchange (lanes l and l+32 share a row); the row
//     sum l is accumulated from the fp32 P, which then goes to 16 bits (round
//     to nearest even) right before the P.V MFMA; m, l and O stay fp32.
//   * the reference max used for exp2 moves -- rescaling O and l by alpha --
//     only when a row's max exceeds it by more than 2^8.  O and l are always
//     relative to the same reference, so O / l is unchanged (the rescale of
//     step 5f is an identity); P stays <= 256, well inside fp16/bf16 range.
//   * causal: the KV loop stops at the block's diagonal; tiles below every
//     row's diagonal take a path with no per-element compare, and on the last
//     tiles each wave skips 32-key subtiles that lie wholly above its rows.
#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"

namespace attn {

namespace {

constexpr int kBM = 128;             // query rows per workgroup
constexpr int kBN = 64;              // key rows per LDS tile
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)
#ifndef ATTN_PF_SETPRIO
#define ATTN_PF_SETPRIO 0  // raise wave priority around MFMA clusters
#endif
#ifndef ATTN_PF_BATCH
#define ATTN_PF_BATCH 0  // read an operand batch from LDS before its MFMAs
#endif

template <int D>
struct PrefillLds {
  static constexpr int KLD = D + 8;      // K row pitch in LDS (elements): 16 B pad, conflict-free reads
  static constexpr int VLD = kBN + 8;    // V^T row pitch in LDS (elements)
  static constexpr int KSZ = kBN * KLD;  // elements per K stage
  static constexpr int VSZ = D * VLD;    // elements per V^T stage
  static constexpr int STAGE = KSZ + VSZ;
};

__device__ __forceinline__ int32_t clamp_bytes(int64_t x) {
  return (int32_t)(x < 0 ? 0 : (x > 0x7fffffff ? 0x7fffffff : x));
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_fwd_kernel(const FwdArgs a) {
  using L = PrefillLds<D>;
  constexpr int KS = D / 16;                 // k-steps of the score MFMA
  constexpr int DT = D / 32;                 // 32-wide head-dim tiles of O
  constexpr int KCH = kBN * D / 8 / 256;     // 16-byte K chunks per thread per tile
  constexpr int VBLK = (kBN / 4) * (D / 8);  // 4-row x 8-col V blocks per tile
  static_assert(VBLK <= 256, "one V block per thread at most");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  // ---- which (batch, q head, query block) this workgroup owns
  const int bid = blockIdx.x;
  int lid = bid;
  if (a.remap) lid = (bid & 7) * (a.nblocks >> 3) + (bid >> 3);  // keep a kv head's blocks on one XCD
  const int per_unit = a.group * a.nqb;
  const int unit = lid / per_unit;
  const int rem = lid - unit * per_unit;
  int qb = rem / a.group;
  const int hg = rem - qb * a.group;
  if (CAUSAL) qb = a.nqb - 1 - qb;  // longest (latest) query blocks first
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int h = kvh * a.group + hg;  // q heads [kvh*group, (kvh+1)*group) share kv head kvh

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;   // this lane's query column within the wave
  const int hh = lane >> 5;  // which half of the wave
  const int q0 = qb * kBM;
  const int qrow = q0 + 32 * w + n;

  // ---- Q fragment, register resident: B operand of S^T = K Q^T (rows >= Nq read as 0)
  u32x4 qf[KS];
  {
    const int64_t qblk = (int64_t)q0 * a.sqn;
    const auto rq = make_rsrc(a.q + (int64_t)b * a.sqb + (int64_t)h * a.sqh + qblk,
                              clamp_bytes(a.q_bytes - 2 * qblk));
    const int32_t qoff = (32 * w + n) * (int32_t)a.sqn * 2 + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = bload16(rq, qoff + 32 * ks) ^ a.qsign;
  }

  const uint16_t* kbase = a.k + (int64_t)b * a.skb + (int64_t)kvh * a.skh;
  const uint16_t* vbase = a.v + (int64_t)b * a.svb + (int64_t)kvh * a.svh;
  const int kv_end = CAUSAL ? min(a.Nkv, q0 + kBM) : a.Nkv;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  // tiles every row of this block sees in full (no mask): below the block's
  // diagonal and before the key tail
  const int n_full = CAUSAL ? min(q0, a.Nkv) / kBN : a.Nkv / kBN;

  // ---- per-thread staging geometry (constant over the loop)
  int32_t koff[KCH];
  int kw[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int id = tid + 256 * i;
    const int row = id / (D / 8), col = id % (D / 8);
    koff[i] = row * (int32_t)a.skn * 2 + 16 * col;
    kw[i] = row * L::KLD + 8 * col;
  }
  const bool vthr = tid < VBLK;
  const int v_kvg = tid % (kBN / 4);  // 4-row group of this thread's V block
  const int v_dc = tid / (kBN / 4);   // 8-column chunk of this thread's V block
  int32_t voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) voff[r] = (4 * v_kvg + r) * (int32_t)a.svn * 2 + 16 * v_dc;
  const int vw = 8 * v_dc * L::VLD + 4 * v_kvg;

  // one KV tile in flight from HBM/L2 to LDS
  struct Staged {
    u32x4 k[KCH];
    u32x4 v[4];
  };
  auto gload = [&](Staged& r, int t) {
    const int64_t ko = (int64_t)t * kBN * a.skn;
    const auto rk = make_rsrc(kbase + ko, clamp_bytes(a.k_bytes - 2 * ko));
#pragma unroll
    for (int i = 0; i < KCH; ++i) r.k[i] = bload16(rk, koff[i]);
    if (vthr) {
      const int64_t vo = (int64_t)t * kBN * a.svn;
      const auto rv = make_rsrc(vbase + vo, clamp_bytes(a.v_bytes - 2 * vo));
#pragma unroll
      for (int q = 0; q < 4; ++q) r.v[q] = bload16(rv, voff[q]);
    }
  };
  auto swrite = [&](const Staged& r, uint16_t* Ks) {
    uint16_t* Vs = Ks + L::KSZ;
#pragma unroll
    for (int i = 0; i < KCH; ++i) store16(Ks + kw[i], r.k[i]);
    if (vthr) {
      // transpose the 4x8 block: V^T row d receives the 4 keys of this group
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 lo{halves<0x05040100u>(r.v[0][j], r.v[1][j]), halves<0x05040100u>(r.v[2][j], r.v[3][j])};
        const u32x2 hi{halves<0x07060302u>(r.v[0][j], r.v[1][j]), halves<0x07060302u>(r.v[2][j], r.v[3][j])};
        *reinterpret_cast<u32x2*>(Vs + vw + (2 * j) * L::VLD) = lo;
        *reinterpret_cast<u32x2*>(Vs + vw + (2 * j + 1) * L::VLD) = hi;
      }
    }
  };

  // ---- online softmax state (fp32): reference max m (log2 domain), this
  //      lane's share of the running sum l, and the O^T accumulator
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;
  const float c = a.c;  // > 0
  // K row fed to MFMA row n: swap bits 2 and 3 so that score register e of a
  // lane holds key 16*(e/8) + 8*hh + e%8 of its 32-key subtile.
  const int sig = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int kr = sig * L::KLD + 8 * hh;
  const int vr = n * L::VLD + 8 * hh;
  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;

  auto compute = [&](const uint16_t* Ks, int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint16_t* Vs = Ks + L::KSZ;
    const int kb = t * kBN;
    bool act1 = true;
    if constexpr (MASKED) {
      if (kb >= a.Nkv || (CAUSAL && kb > wq_hi)) return;  // whole tile above this wave's rows
      act1 = kb + 32 < a.Nkv && (!CAUSAL || kb + 32 <= wq_hi);
    }
    // S^T = K Q^T for the two 32-key subtiles
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#if ATTN_PF_SETPRIO
    __builtin_amdgcn_s_setprio(1);
#endif
#if ATTN_PF_BATCH
    {
      u32x4 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = load16(Ks + kr + 16 * ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s0 = mfma_32x32x16<BF16>(kf[ks], qf[ks], s0);
    }
    if (act1) {
      u32x4 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = load16(Ks + 32 * L::KLD + kr + 16 * ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s1 = mfma_32x32x16<BF16>(kf[ks], qf[ks], s1);
    }
#else
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s0 = mfma_32x32x16<BF16>(load16(Ks + kr + 16 * ks), qf[ks], s0);
    if (act1) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s1 = mfma_32x32x16<BF16>(load16(Ks + 32 * L::KLD + kr + 16 * ks), qf[ks], s1);
    }
#endif
#if ATTN_PF_SETPRIO
    __builtin_amdgcn_s_setprio(0);
#endif
    if constexpr (MASKED) {
      // mask before the row max: key index of register e is kb + 16*(e/8) + 8*hh + e%8
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kv0 = kb + 16 * (e >> 3) + 8 * hh + (e & 7);
        const int kv1 = kv0 + 32;
        const bool vis0 = kv0 < a.Nkv && (!CAUSAL || kv0 <= qrow);
        const bool vis1 = act1 && kv1 < a.Nkv && (!CAUSAL || kv1 <= qrow);
        s0[e] = vis0 ? s0[e] : -INFINITY;
        s1[e] = vis1 ? s1[e] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = vmax(mx, vmax(s0[e], s1[e]));
    mx = max_xor32(mx) * c;  // this row's max in the log2 domain

    // move the reference max only when some row's max outgrew it by > 2^8
    if (__any(mx > m + kRescaleLog2)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      l *= alpha;
      m = m_new;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;  // rows with nothing visible yet get P = 0

    // P = exp2(s*c - m) in fp32, its fp32 row sum, then the 16-bit B operand of P.V
    u32x4 pf[4];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s0[e], c, -m_use));
      const float p1 = fast_exp2(__builtin_fmaf(s0[e + 1], c, -m_use));
      const float p2 = fast_exp2(__builtin_fmaf(s1[e], c, -m_use));
      const float p3 = fast_exp2(__builtin_fmaf(s1[e + 1], c, -m_use));
      rs0 += p0 + p1;
      rs1 += p2 + p3;
      pf[e >> 3][(e & 7) >> 1] = pack2<BF16>(p0, p1);
      pf[2 + (e >> 3)][(e & 7) >> 1] = pack2<BF16>(p2, p3);
    }
    l += rs0 + rs1;

    // O^T += V^T P^T : A = V^T rows from LDS, B = P^T from registers
#if ATTN_PF_SETPRIO
    __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 2 || act1) {
#if ATTN_PF_BATCH
        u32x4 vf[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt] = load16(Vs + 32 * dt * L::VLD + vr + 16 * kk);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma_32x32x16<BF16>(vf[dt], pf[kk], oacc[dt]);
#else
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = mfma_32x32x16<BF16>(load16(Vs + 32 * dt * L::VLD + vr + 16 * kk), pf[kk], oacc[dt]);
#endif
      }
    }
#if ATTN_PF_SETPRIO
    __builtin_amdgcn_s_setprio(0);
#endif
  };
  using full_t = std::false_type;
  using mask_t = std::true_type;
  uint16_t* const S0 = smem;
  uint16_t* const S1 = smem + L::STAGE;

  // ---- KV loop, double-buffered LDS: the global loads of tile t+1 are issued
  //      before tile t is computed.  Full tiles go in pairs (stage 0, stage 1);
  //      the remaining tiles (diagonal / key tail) take the masked path.
  Staged rs;
  if (ntiles > 0) {
    gload(rs, 0);
    swrite(rs, S0);
  }
  __syncthreads();
  int t = 0;
  for (; t + 1 < n_full; t += 2) {
    gload(rs, t + 1);
    compute(S0, t, full_t{});
    swrite(rs, S1);
    __syncthreads();
    if (t + 2 < ntiles) gload(rs, t + 2);
    compute(S1, t + 1, full_t{});
    if (t + 2 < ntiles) swrite(rs, S0);
    __syncthreads();
  }
  for (; t < ntiles; ++t) {
    const bool odd = t & 1;
    if (t + 1 < ntiles) gload(rs, t + 1);
    compute(odd ? S1 : S0, t, mask_t{});
    if (t + 1 < ntiles) swrite(rs, odd ? S0 : S1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, cast, store; lse = (m + log2 l) ln 2
  l = sum_xor32(l);
  if (qrow < a.Nq) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    uint16_t* op = a.o + (int64_t)b * a.sob + (int64_t)h * a.soh + (int64_t)qrow * a.son;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hh;
        const u32x2 v2{pack2<BF16>(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                       pack2<BF16>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = v2;
      }
    }
    if (a.lse != nullptr && hh == 0)
      a.lse[((int64_t)b * a.Hq + h) * a.Nq + qrow] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, CAUSAL>), dim3(a.nblocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_c(const FwdArgs& a, bool causal, hipStream_t stream) {
  return causal ? launch_t<D, BF16, true>(a, stream) : launch_t<D, BF16, false>(a, stream);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, bool bf16, bool causal, hipStream_t stream) {
  return bf16 ? launch_c<D, true>(a, causal, stream) : launch_c<D, false>(a, causal, stream);
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, bool causal, hipStream_t stream) {
  if (D == 64) return launch_d<64>(a, bf16, causal, stream);
  return launch_d<128>(a, bf16, causal, stream);
}

}  // namespace attn
