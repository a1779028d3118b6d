// Device-side helpers shared by the DSA sparse-prefill kernels (gfx950 / CDNA4).
//
// Wave64 throughout.  MFMA operand layouts used by the kernels (lane l of a wave):
//   16x16x32 bf16  A: row l%16, k-chunk 8*(l/16)..+8     B: col l%16, same k-chunk
//                  C: rows 4*(l/16)+j (j = 0..3), col l%16
//   16x16x16 bf16  A: row l%16, k 4*(l/16)..+4           B: col l%16, same k
// A dot product is invariant under any relabelling of k that A and B share, so
// only the row/column placement and the C layout above matter for correctness.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite or +-inf)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, ((uint32_t)b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Blocks are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Remap so that every XCD receives a contiguous range of logical block ids:
// neighbouring work items then share that XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8;
  const int x = b % 8, k = b / 8;
  const int start = (x < r) ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return start + k;
}

// max / sum over the 4 lanes l, l^16, l^32, l^48 (the 4 row groups of a 16x16 C tile)
__device__ __forceinline__ float max_over_rowgroups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float sum_over_rowgroups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace dsa
