// LDS tile helpers shared by the prefill and backward kernels (gfx950 only):
// the XOR swizzle of row-major K/V (or Q/dO) tiles, transposing and plain LDS
// reads, buffer-to-LDS loads issued as inline assembly, whole-row stores of an
// accumulator tile through LDS, and a fence-free workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_common.hpp"

namespace attn {

// XOR swizzle of the 16-byte slots of K/V row `row` in LDS (slot = chunk ^
// swz(row)).  With 256 bytes of banks served per LDS cycle it keeps three
// access patterns free of bank conflicts with no padding:
//   * the DMA writes: 1 KiB contiguous per wave;
//   * the K operand reads (16 bytes a lane, 16 lanes a cycle): 16 rows at one
//     chunk, so swz must take distinct values on any 16 rows sharing their
//     256-byte bank phase;
//   * the transposed V reads (8 bytes a lane, 32 lanes a cycle): 4 consecutive
//     rows (from a multiple of 4) x 4 consecutive chunks (from a multiple of
//     4), so the rows that share a bank phase must land in different groups of
//     4 slots.
// D = 128 (256-byte rows): bits 2-3 of swz are row % 4, bits 0-1 are row/4 % 4.
// D = 64 (128-byte rows, two per bank phase; rows of one parity share it): with
// x = row/2 % 8, bit 2 of swz is x % 2 and bits 0-1 are x/2 % 4.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
}

__device__ __forceinline__ int32_t clamp_bytes(int64_t x) {
  return (int32_t)(x < 0 ? 0 : (x > 0x7fffffff ? 0x7fffffff : x));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// 4 x 16-bit from LDS byte address `addr`, transposed across each group of 16
// lanes: lane i of a group receives element i % 4 of the 8-byte pieces
// addressed by lanes 4r + i/4 (r = 0..3) of its group.
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// 16 bytes from LDS byte address `addr`
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr) { return *(lds_u32x4*)(uintptr_t)addr; }

// 8 bytes to LDS byte address `addr`
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ void lds_store8(uint32_t addr, u32x2 v) { *(lds_u32x2*)(uintptr_t)addr = v; }

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t*)p;
}

// an LDS address the compiler may not see through: keeps a per-lane base
// address whole in its register, so that only the (< 64 KiB) stage and
// sub-tile offsets are folded into the instructions' immediate offsets (the
// mask tells it the address is small and non-negative, which that folding
// requires)
__device__ __forceinline__ uint32_t opaque_lds(uint32_t x) {
  asm("" : "+v"(x));
  return x & 0x3ffff;
}

// buffer resource words (raw, unswizzled, range-checked against `bytes`) for
// the inline-assembly loads below; every field is made wave-uniform
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4{(int)__builtin_amdgcn_readfirstlane((uint32_t)p),
               (int)(__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffff),
               (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes), 0x00020000};
}

// one 16-byte global load per lane straight into LDS: lane l's data lands at
// LDS byte address lds_base + 16 l (lds_base wave-uniform, passed in m0);
// loads at or past the resource's range write zeros.  Issued as inline
// assembly so that the compiler does not track it as a pending LDS write: its
// tracking would put a wait for every such load in flight (including the ones
// for tiles needed later) in front of the transposing LDS reads and of any
// fenced barrier.  The ring's explicit vmcnt waits and barriers order it.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t lds_base, int32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds_base));
}

// Stores a wave's 32 x D tile of 16-bit values as whole rows.  The tile is a
// transposed-MFMA accumulator: lane (n, hh) = (l % 32, l / 32) holds row n,
// columns 32 dt + 8 g + 4 hh + j in acc[dt][4 g + j]; each value is
// multiplied by `mul` (the lane's own factor) and rounded to 16 bits.
// Stored directly, every instruction would touch 32 rows in 8-byte pieces;
// instead the tile goes through `stg`, 32 * 2D bytes of LDS that no other
// wave uses meanwhile, and back as 16-byte chunks of whole rows, 4 (D = 128)
// or 8 (D = 64) rows per instruction.  Rows r with row0 + r < nrows go to
// base + (row0 + r) * stride.  The 8-byte piece s of row r sits at slot
// s ^ X(r), X(r) = r mod 32 (D = 128, a row per 256 bytes of banks) or
// r/2 mod 16 (D = 64, two rows per 256 bytes): the 32 rows' pieces of one
// write fill all 64 banks, and a 16-byte chunk c then sits at c ^ X(r)/2,
// its halves swapped when X(r) is odd, so the row reads are conflict free.
template <int D, bool BF16>
__device__ __forceinline__ void store_tile_rows(uint32_t stg, const f32x16 (&acc)[D / 32], float mul, uint16_t* base,
                                                int64_t stride, int row0, int nrows) {
  constexpr int RB = 2 * D;      // bytes per row
  constexpr int CPR = RB / 16;   // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per 64-lane read
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  auto xs = [](int r) { return D == 128 ? (r & 31) : ((r >> 1) & 15); };
  {
    const int n = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 4 * dt + g;
        const u32x2 v2{pack2<BF16>(acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul),
                       pack2<BF16>(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul)};
        lds_store8(stg + n * RB + 8 * ((2 * c + hh) ^ xs(n)), v2);
      }
  }
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / CPR, c = lane % CPR;
    u32x4 v4 = lds_load16(stg + r * RB + 16 * (c ^ (xs(r) >> 1)));
    if (xs(r) & 1) v4 = u32x4{v4[2], v4[3], v4[0], v4[1]};
    if (row0 + r < nrows) store16(base + (int64_t)(row0 + r) * stride + 8 * c, v4);
  }
}

// workgroup barrier without a memory fence: a tile's loads are waited for
// (vmcnt) before the barrier that publishes it, and every wave has consumed
// all of its LDS reads of a stage before the barrier after which that stage
// is refilled.  The clobber keeps the compiler from moving memory accesses
// across it, the scheduling barriers every other instruction.
__device__ __forceinline__ void barrier_nofence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace attn
