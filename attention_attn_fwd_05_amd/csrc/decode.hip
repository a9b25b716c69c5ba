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
//     one contiguous chunk ("split") of the cache.
//   * 128-key tiles are staged in LDS (K row-major, V transposed), double
//     buffered; each wave takes 32 keys of a tile.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32; the q heads of the
//     group are the 16 MFMA columns.  K rows are fed in a permuted order so the
//     score registers are directly the B operand of the P.V MFMA.
//   * each workgroup merges its 4 waves' (m, l, o) in LDS; with one split it
//     writes the normalised output, otherwise it stores its partial and the
//     last workgroup of the (batch, kv head, head group) to arrive -- counted
//     with a device-scope atomic ticket -- merges all partials with the same
//     max/rescale identity and resets the ticket to zero.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace attn {

namespace {

constexpr int kDT = 128;  // keys per LDS tile (32 per wave)

template <int D>
struct DecodeLds {
  static constexpr int KLD = D + 8;
  static constexpr int VLD = kDT + 8;
  static constexpr int KSZ = kDT * KLD;
  static constexpr int VSZ = D * VLD;
  static constexpr int STAGE = KSZ + VSZ;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256, 1) void decode_kernel(const DecodeArgs a) {
  using L = DecodeLds<D>;
  constexpr int KS = D / 32;                  // k-steps of the score MFMA
  constexpr int NDT = D / 16;                 // 16-wide head-dim tiles of O
  constexpr int KCH = kDT * D / 8 / 256;      // 16-byte K chunks per thread per tile
  constexpr int VBLK = (kDT / 4) * (D / 8);   // 4x8 V blocks per tile
  constexpr int VPT = VBLK / 256;             // V blocks per thread
  static_assert(VBLK % 256 == 0, "V blocks divide evenly");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int split = blockIdx.x;
  const int hgi = blockIdx.y;
  const int unit = blockIdx.z;
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int h0 = kvh * a.group + hgi * a.heads_per_wg;  // first q head of this workgroup
  const int nh = min(a.heads_per_wg, a.group - hgi * a.heads_per_wg);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane & 15;  // MFMA column = q head within the group
  const int rg = lane >> 4;   // 4-row group of the MFMA output / k-group of operands

  const int k0 = split * a.rows_per_split;
  const int k1 = min(a.cache_len, k0 + a.rows_per_split);
  const int ntiles = (k1 - k0 + kDT - 1) / kDT;

  // q heads as the B operand (columns beyond nh are zero)
  u32x4 qf[KS];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.sqb + (int64_t)(h0 + col) * a.sqh;
    const bool ok = col < nh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = ok ? load16(qp + 32 * ks + 8 * rg) : u32x4{0, 0, 0, 0};
      qf[ks] = x ^ a.qsign;
    }
  }

  const uint16_t* kp = a.k + (int64_t)b * a.skb + (int64_t)kvh * a.skh;
  const uint16_t* vp = a.v + (int64_t)b * a.svb + (int64_t)kvh * a.svh;

  u32x4 kreg[KCH];
  u32x4 vreg[VPT][4];
  auto gload = [&](int t) {
    const int kb = k0 + t * kDT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int row = id / (D / 8), c8 = id % (D / 8);
      kreg[i] = (kb + row < k1) ? load16(kp + (int64_t)(kb + row) * a.skn + 8 * c8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int id = tid + 256 * j;
      const int kvg = id % (kDT / 4), dc = id / (kDT / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = kb + 4 * kvg + r;
        vreg[j][r] = (row < k1) ? load16(vp + (int64_t)row * a.svn + 8 * dc) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto swrite = [&](int buf) {
    uint16_t* Ks = smem + buf * L::STAGE;
    uint16_t* Vs = Ks + L::KSZ;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int row = id / (D / 8), c8 = id % (D / 8);
      store16(Ks + row * L::KLD + 8 * c8, kreg[i]);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int id = tid + 256 * j;
      const int kvg = id % (kDT / 4), dc = id / (kDT / 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t x0 = (vreg[j][0][e >> 1] >> sh) & 0xffffu;
        const uint32_t x1 = (vreg[j][1][e >> 1] >> sh) & 0xffffu;
        const uint32_t x2 = (vreg[j][2][e >> 1] >> sh) & 0xffffu;
        const uint32_t x3 = (vreg[j][3][e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<u32x2*>(Vs + (8 * dc + e) * L::VLD + 4 * kvg) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
      }
    }
  };

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{};
  float m = -INFINITY;  // running max of this lane's head column (log2 domain)
  float l = 0.f;        // this lane's share of the running sum
  const float c = a.c;
  // MFMA row i of key group gi reads key 8*(i/4) + 4*gi + i%4 of the wave's 32,
  // so that lane (col, rg) holds keys 8*rg .. 8*rg+7 in its score registers.
  const int krow0 = 32 * w + 8 * (col >> 2) + (col & 3);

  auto compute = [&](int t, int buf) {
    const int kb = k0 + t * kDT + 32 * w;  // first key of this wave
    if (kb >= k1) return;
    const uint16_t* Ks = smem + buf * L::STAGE;
    const uint16_t* Vs = Ks + L::KSZ;
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma_16x16x32<BF16>(load16(Ks + krow0 * L::KLD + 32 * ks + 8 * rg), qf[ks], s0);
      s1 = mfma_16x16x32<BF16>(load16(Ks + (krow0 + 4) * L::KLD + 32 * ks + 8 * rg), qf[ks], s1);
    }
    // lane (col, rg): s0[e] is key kb + 8*rg + e, s1[e] is key kb + 8*rg + 4 + e
    float mx = -INFINITY;
    const bool full = kb + 32 <= k1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!full) {
        const int key = kb + 8 * rg + e;
        s0[e] = (key < k1) ? s0[e] * c : -INFINITY;
        s1[e] = (key + 4 < k1) ? s1[e] * c : -INFINITY;
      } else {
        s0[e] *= c;
        s1[e] *= c;
      }
      mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = fast_exp2(s0[e] - m_use);
      p[4 + e] = fast_exp2(s1[e] - m_use);
    }
    l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    m = m_new;
    const u32x4 pf{pack2<BF16>(p[0], p[1]), pack2<BF16>(p[2], p[3]), pack2<BF16>(p[4], p[5]),
                   pack2<BF16>(p[6], p[7])};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      oacc[dt] *= alpha;
      oacc[dt] = mfma_16x16x32<BF16>(load16(Vs + (16 * dt + col) * L::VLD + 32 * w + 8 * rg), pf, oacc[dt]);
    }
  };

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

  // ---- merge the 4 waves in LDS: per wave m[16], l[16], o[16][D] (fp32)
  float* red = reinterpret_cast<float*>(smem);
  float* rm = red;                 // [4][16]
  float* rl = red + 64;            // [4][16]
  float* ro = red + 128;           // [4][16][D]
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (rg == 0) {
    rm[w * 16 + col] = m;
    rl[w * 16 + col] = l;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) ro[(w * 16 + col) * D + 16 * dt + 4 * rg + e] = oacc[dt][e];
  __syncthreads();

  // thread -> (head hn, 8-wide slice of the head dim)
  constexpr int SL = D / 16;  // elements per thread
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
    for (int j = 0; j < SL; ++j) acc[j] += sc * ro[(ww * 16 + hn) * D + d0 + j];
  }

  auto store_out = [&](float Mx, float Lx, const float* o) {
    if (hn >= nh) return;
    const float inv = (Lx > 0.f) ? 1.f / Lx : 0.f;
    uint16_t* op = a.o + (int64_t)b * a.sob + (int64_t)(h0 + hn) * a.soh + d0;
    if constexpr (SL == 8) {
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = pack2<BF16>(o[2 * j] * inv, o[2 * j + 1] * inv);
      store16(op, v);
    } else {
      static_assert(SL == 4, "D is 64 or 128");
      *reinterpret_cast<u32x2*>(op) = u32x2{pack2<BF16>(o[0] * inv, o[1] * inv), pack2<BF16>(o[2] * inv, o[3] * inv)};
    }
    if (a.lse != nullptr && (tid & 15) == 0)
      a.lse[(int64_t)b * a.Hq + h0 + hn] = (Lx > 0.f) ? (Mx + __log2f(Lx)) * kLn2 : -INFINITY;
  };

  if (a.nsplit == 1) {
    store_out(M, Ls, acc);
    return;
  }

  // ---- several splits: publish this split's partial, the last arrival merges
  const int64_t slot = ((int64_t)unit * a.hgroups + hgi);
  const int64_t pstride = (int64_t)a.heads_per_wg * (D + 2);
  float* mypart = a.part + (slot * a.nsplit + split) * pstride;
  if (hn < nh) {
    float* pr = mypart + (int64_t)hn * (D + 2);
    if ((tid & 15) == 0) {
      pr[0] = M;
      pr[1] = Ls;
    }
#pragma unroll
    for (int j = 0; j < SL; ++j) pr[2 + d0 + j] = acc[j];
  }
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.tickets + slot, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (uint32_t)(a.nsplit - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (hn < nh) {
    const float* base = a.part + slot * a.nsplit * pstride + (int64_t)hn * (D + 2);
    float Mg = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) Mg = fmaxf(Mg, base[s * pstride]);
    const float Mgu = (Mg == -INFINITY) ? 0.f : Mg;
    float Lg = 0.f;
    float og[SL];
#pragma unroll
    for (int j = 0; j < SL; ++j) og[j] = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float* pr = base + s * pstride;
      const float sc = fast_exp2(pr[0] - Mgu);
      Lg += sc * pr[1];
#pragma unroll
      for (int j = 0; j < SL; ++j) og[j] += sc * pr[2 + d0 + j];
    }
    store_out(Mg, Lg, og);
  }
  if (tid == 0) __hip_atomic_store(a.tickets + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool BF16>
hipError_t launch_t(const DecodeArgs& a, int B, hipStream_t stream) {
  using L = DecodeLds<D>;
  const size_t lds = 2 * L::STAGE * sizeof(uint16_t);
  // allow more than the default dynamic LDS (gfx950 has 160 KiB per CU); set once per device
  static bool attr_set[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<D, BF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  dim3 grid(a.nsplit, a.hgroups, B * a.Hkv);
  hipLaunchKernelGGL((decode_kernel<D, BF16>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
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

}  // namespace

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
