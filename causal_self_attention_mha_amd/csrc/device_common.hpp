// Device-side building blocks for the gfx950 attention kernels: bf16 vector
// types, MFMA wrappers, conversions and wavefront (64-lane) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace na {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on one wavefront.
// Operand lanes: A row m and B column n live in lane (m or n) mod 32; each
// lane holds 8 consecutive-k values of its half (lanes 32..63 hold the other
// half of k).  Result: lane l, element r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16.
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Pack two fp32 values into one dword of two bf16 (lo first).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = to_bf16(lo), b = to_bf16(hi);
  u16 ua = __builtin_bit_cast(u16, a), ub = __builtin_bit_cast(u16, b);
  return static_cast<uint32_t>(ua) | (static_cast<uint32_t>(ub) << 16);
}

// Sum over all 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum over aligned groups of 16 lanes.
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sixteen-byte global/LDS load and store through a 4 x dword vector.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// The row of a 32-key (or 32-query) block that lane l (mod 32) loads as the
// A operand of the score MFMA, chosen so that accumulator element r of lane l
// ends up holding block row 8*(l/32) + (r%8) + 16*(r/8).  That makes each
// group of 8 accumulator elements a contiguous run of 8 rows, which is exactly
// one lane's share of a 16-row k-chunk of the following MFMA.  It swaps bits
// 2 and 3 of m.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Block row held by accumulator element r of lane l after a perm_row-loaded
// score MFMA.
__device__ __forceinline__ int acc_row(int lane, int r) {
  return 8 * (lane >> 5) + (r & 7) + 16 * (r >> 3);
}

}  // namespace na
