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
//     32 rows for the whole KV loop.
//   * KV tiles of 64 rows are staged in LDS, double buffered: K row-major, V
//     transposed (head-dim major) so both MFMA operands are single 16-byte LDS
//     reads.  Global loads for tile t+1 are issued before tile t is computed.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//     Q is the register-resident B operand and each lane ends up owning one
//     query row's scores.  The K rows fed to the MFMA are permuted (bits 2 and
//     3 of the row index swapped) so that the fp32 score registers of a lane
//     are exactly the B operand layout of the P.V MFMA: no data movement
//     between the two contractions.
//   * online softmax in the log2 domain: t = s * scale * log2(e); the row max
//     needs one cross-lane exchange (lanes l and l+32 share a row); P goes to
//     16 bits with round-to-nearest-even right before the P.V MFMA; m, l and
//     the O accumulator stay fp32.  O is rescaled by alpha only when some row
//     of the wave changed its max (alpha == 1 otherwise: skipping is exact).
//   * causal: the KV loop stops at the block's diagonal, subtiles wholly above
//     a wave's diagonal are skipped, and the per-element compare runs only on
//     tiles that straddle the diagonal or the KV tail.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace attn {

namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // key rows per LDS tile

template <int D>
struct PrefillLds {
  static constexpr int KLD = D + 8;      // K row pitch in LDS (elements): 16 B pad, conflict-free reads
  static constexpr int VLD = kBN + 8;    // V^T row pitch in LDS (elements)
  static constexpr int KSZ = kBN * KLD;  // elements per K stage
  static constexpr int VSZ = D * VLD;    // elements per V^T stage
  static constexpr int STAGE = KSZ + VSZ;
};

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

  // ---- Q fragment, register resident: B operand of S^T = K Q^T
  u32x4 qf[KS];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.sqb + (int64_t)h * a.sqh + (int64_t)qrow * a.sqn;
    const bool ok = qrow < a.Nq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = ok ? load16(qp + 16 * ks + 8 * hh) : u32x4{0, 0, 0, 0};
      qf[ks] = x ^ a.qsign;
    }
  }

  const uint16_t* kp = a.k + (int64_t)b * a.skb + (int64_t)kvh * a.skh;
  const uint16_t* vp = a.v + (int64_t)b * a.svb + (int64_t)kvh * a.svh;
  const int kv_end = CAUSAL ? min(a.Nkv, q0 + kBM) : a.Nkv;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- global -> register staging of one KV tile
  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int v_kvg = tid % (kBN / 4);  // 4-row group of this thread's V block
  const int v_dc = tid / (kBN / 4);   // 8-column chunk of this thread's V block
  auto gload = [&](int t) {
    const int kb = t * kBN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int row = id / (D / 8), col = id % (D / 8);
      kreg[i] = (kb + row < a.Nkv) ? load16(kp + (int64_t)(kb + row) * a.skn + 8 * col) : u32x4{0, 0, 0, 0};
    }
    if (tid < VBLK) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = kb + 4 * v_kvg + r;
        vreg[r] = (row < a.Nkv) ? load16(vp + (int64_t)row * a.svn + 8 * v_dc) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto swrite = [&](int buf) {
    uint16_t* Ks = smem + buf * L::STAGE;
    uint16_t* Vs = Ks + L::KSZ;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int row = id / (D / 8), col = id % (D / 8);
      store16(Ks + row * L::KLD + 8 * col, kreg[i]);
    }
    if (tid < VBLK) {
      // transpose the 4x8 block: V^T row d gets the 4 keys of this group
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t x0 = (vreg[0][e >> 1] >> sh) & 0xffffu;
        const uint32_t x1 = (vreg[1][e >> 1] >> sh) & 0xffffu;
        const uint32_t x2 = (vreg[2][e >> 1] >> sh) & 0xffffu;
        const uint32_t x3 = (vreg[3][e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<u32x2*>(Vs + (8 * v_dc + e) * L::VLD + 4 * v_kvg) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
      }
    }
  };

  // ---- online softmax state (fp32): running max m (log2 domain), this lane's
  //      share of the running sum l, and the O^T accumulator
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;
  const float c = a.c;
  // K row fed to MFMA row n: swap bits 2 and 3 so that score register e of a
  // lane holds key 16*(e/8) + 8*hh + e%8 of its 32-key subtile.
  const int sig = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;

  auto compute = [&](int t, int buf) {
    const int kb = t * kBN;
    const bool act0 = kb < a.Nkv && (!CAUSAL || kb <= wq_hi);
    if (!act0) return;  // the whole tile is above this wave's diagonal
    const bool act1 = kb + 32 < a.Nkv && (!CAUSAL || kb + 32 <= wq_hi);
    const bool need_mask = (kb + kBN > a.Nkv) || (CAUSAL && kb + kBN - 1 > wq_lo);
    const uint16_t* Ks = smem + buf * L::STAGE;
    const uint16_t* Vs = Ks + L::KSZ;

    // S^T = K Q^T for the two 32-key subtiles
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s0 = mfma_32x32x16<BF16>(load16(Ks + sig * L::KLD + 16 * ks + 8 * hh), qf[ks], s0);
    if (act1) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s1 = mfma_32x32x16<BF16>(load16(Ks + (32 + sig) * L::KLD + 16 * ks + 8 * hh), qf[ks], s1);
    }

    // row max of the scaled scores (mask first, then reduce)
    float mx = -INFINITY;
    if (!need_mask) {
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
      mx *= c;
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kv0 = kb + 16 * (e >> 3) + 8 * hh + (e & 7);
        const int kv1 = kv0 + 32;
        const bool vis0 = kv0 < a.Nkv && (!CAUSAL || kv0 <= qrow);
        const bool vis1 = act1 && kv1 < a.Nkv && (!CAUSAL || kv1 <= qrow);
        s0[e] = vis0 ? s0[e] * c : -INFINITY;
        s1[e] = vis1 ? s1[e] * c : -INFINITY;
        mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // a row with nothing visible yet
    const float alpha = fast_exp2(m - m_use);

    // P = exp2(t - m), its row sum, and the 16-bit B operand of P.V
    u32x4 pf[4];
    float rs = 0.f;
    if (!need_mask) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s0[e], c, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s0[e + 1], c, -m_use));
        const float p2 = fast_exp2(__builtin_fmaf(s1[e], c, -m_use));
        const float p3 = fast_exp2(__builtin_fmaf(s1[e + 1], c, -m_use));
        rs += (p0 + p1) + (p2 + p3);
        pf[(e >> 3)][(e & 7) >> 1] = pack2<BF16>(p0, p1);
        pf[2 + (e >> 3)][(e & 7) >> 1] = pack2<BF16>(p2, p3);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(s0[e] - m_use);
        const float p1 = fast_exp2(s0[e + 1] - m_use);
        const float p2 = fast_exp2(s1[e] - m_use);
        const float p3 = fast_exp2(s1[e + 1] - m_use);
        rs += (p0 + p1) + (p2 + p3);
        pf[(e >> 3)][(e & 7) >> 1] = pack2<BF16>(p0, p1);
        pf[2 + (e >> 3)][(e & 7) >> 1] = pack2<BF16>(p2, p3);
      }
    }
    l = l * alpha + rs;
    m = m_new;

    // alpha rescale of the accumulator before adding this tile's P.V
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }

    // O^T += V^T P^T : A = V^T rows from LDS, B = P^T from registers
    const int nk = act1 ? 4 : 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < nk) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = mfma_32x32x16<BF16>(load16(Vs + (32 * dt + n) * L::VLD + 16 * kk + 8 * hh), pf[kk], oacc[dt]);
      }
    }
  };

  // ---- KV loop, double-buffered LDS
  if (ntiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    compute(t, buf);
    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, cast, store; lse = (m + log2 l) ln 2
  l += __shfl_xor(l, 32);
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
