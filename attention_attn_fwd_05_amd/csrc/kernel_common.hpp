// Device-side helpers shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16) * B(16x32), 16-bit inputs.  Lane l supplies
// A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; element e of the result
// in lane l is D[8*(e/4) + 4*(l/32) + e%4][l%32].
template <bool BF16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8*(l/16) .. +7]
// and B[8*(l/16) .. +7][l%16]; element e of the result in lane l is
// D[4*(l/16) + e][l%16].
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two 16-bit values (round to nearest even) in one dword,
// `lo` in the low half (one v_cvt_pk_{f16,bf16}_f32 on gfx950).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// max / sum of x over lanes l and l ^ 32 (l ^ 16) with v_permlane32_swap
// (v_permlane16_swap), gfx950: with x as both operands the two results hold,
// in every lane, the values of lanes l and l ^ 32 (l ^ 16), so combining them
// is the exchange; VALU operations, where a shuffle would be an LDS round trip.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// max / sum of x over all 64 lanes, the same value in every lane.  Inside each
// row of 16 lanes DPP moves combine neighbours (quad_perm [1,0,3,2]), pairs
// (quad_perm [2,3,0,1]), the two quads of each half-row (row_half_mirror: after
// the first two steps every lane of a quad holds the quad's result, so lane i
// meeting lane 7 - i combines the two quads) and the two half-rows (row_mirror,
// likewise); the permlane swaps above then combine the four rows.  Every step
// is commutative per lane pair, so all lanes end with bitwise the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return sum_xor32(sum_xor16(x));
}

// Buffer resource over [base, base + bytes): 16-byte loads at byte offsets
// >= bytes return zeros (hardware range check), so ragged tails need no branch.
// `base` and `bytes` must be wave-uniform; readfirstlane makes that explicit to
// the compiler, which then keeps the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* const pu = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// the same with the non-temporal hint: data read once (a decode's K/V stream)
// is not kept in the caches at the expense of other lines
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// Low (SEL = 0x05040100) or high (SEL = 0x07060302) 16-bit halves of two dwords:
// result = {a.half, b.half} with a's half in the low 16 bits.
template <uint32_t SEL>
__device__ __forceinline__ uint32_t halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, SEL);
}

template <bool BF16>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (BF16)
    return __builtin_bit_cast(float, bits16 << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + (low half + high half) of a dword holding two bf16 values, summed in
// fp32 (one v_dot2c_f32_bf16 against (1, 1); the products are exact)
__device__ __forceinline__ float sum2_bf16(uint32_t two, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, two), __builtin_bit_cast(bf16x2, 0x3F803F80u), acc,
                                         false);
}

// NaN-propagating maximum (v_maximum3_f32 on gfx950): unlike fmaxf it needs no
// quieting of its inputs, which matters in a row max over many scores.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace attn
