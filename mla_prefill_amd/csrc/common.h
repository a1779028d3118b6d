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

// A wave-uniform value or pointer, proven so to the compiler: loads through a
// uniform pointer become scalar loads (counted in lgkmcnt, not vmcnt).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// Read-only global data addressed uniformly by a wave: a pointer into the
// constant address space (the data is never written while a kernel runs), so
// its loads go through the scalar cache.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ const_i32* uniform_const(const int32_t* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const_i32*)(((uint64_t)hi << 32) | lo);
}

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

// 32x32x16 bf16: A lane l = row l%32, k-chunk 8*(l/32)..+8; B = col l%32, same chunk;
// C register j = row 8*(j/4) + 4*(l/32) + j%4, col l%32.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same 32x32x16 MFMA written out, with its accumulator in VGPRs: score accumulators that
// the softmax reads and masks in place stay out of the accumulation registers, which the O^T
// accumulators fill.  The compiler sees no latency for these, so a VALU read of the result
// must come several MFMAs later (the kernels keep at least four between them).
__device__ __forceinline__ f32x16 mfma_qk_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ f32x16 mfma_qk(bf16x8 a, bf16x8 b, f32x16 c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}

// ---------------------------------------------------------------------------
// Asynchronous global -> LDS copies (gfx950 LDS DMA).
//
// One instruction per wave: lane l copies `size` bytes from its own global
// address to lds_base + l * size, where lds_base is wave-uniform.  The copies
// count in vmcnt like any vector load; the kernels wait for them with
// wait_vmcnt<N>() (N = vector-memory operations issued after the ones needed)
// and then a workgroup barrier before other waves read the data (or, for a
// wave reading its own copies, wait_vmcnt_dep, which orders the reads by a
// data dependency).  They are written as inline asm so that the compiler does
// not serialize the pipeline with a full vmcnt(0) before every LDS read; the
// kernels that use them issue no other vector-memory loads inside their
// pipelined loops, and use no dynamic register indexing (the copies set M0).
// The copies only write LDS, so they carry no "memory" clobber: that keeps
// loads of read-only global data eligible for the scalar cache.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const lds_u8*)p);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is named as clobbered on purpose
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "m0");
}

// The same copy addressed as a uniform base plus this lane's 32-bit byte offset (below 2^31):
// line offsets can live in the base, so the lanes need no address arithmetic per line.
__device__ __forceinline__ void dma16_sbase(uint32_t lane_ofs, const void* base, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_ofs), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "m0");
}

__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "m0");
}

// Compiler-only fence: keeps the scheduler from hoisting LDS operand reads of
// later MFMA groups above it (bounds the registers held by in-flight reads).
__device__ __forceinline__ void sched_fence() { asm volatile("" : : : "memory"); }

// Opaque to the optimizer: a value passed through here is recomputed inside a
// loop instead of being hoisted (hoisted per-lane offsets otherwise spill).
template <typename T>
__device__ __forceinline__ T loop_local(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait as above and return `x` unchanged; LDS addresses computed from the
// result cannot be read before the wait.
template <int N>
__device__ __forceinline__ int wait_vmcnt_dep(int x) {
  asm volatile("s_waitcnt vmcnt(%1)" : "+v"(x) : "n"(N));
  return x;
}

// transposed 64-bit LDS read (gfx950).  Within each group of 16 lanes, output
// lane i slot j receives slot i%4 of the 4 elements addressed by lane i/4 + 4j
// of that group.
__device__ __forceinline__ u16x4 lds_read_tr16(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((const lds_u8*)p));
  return __builtin_bit_cast(u16x4, v);
}

// ---------------------------------------------------------------------------
// LDS tile layout for row-gathered operands ("8-row groups"):
//   rows are stored in groups of 8; within a group, 16-byte chunk k of row r
//   lives in 1 KiB block k / 8 at 128 B * (r % 8) + 16 B * pos, with
//   pos = (k % 8) ^ swz8(r % 8) ^ (r / 8 % 8).
// One wave copy (64 lanes x 16 B) fills one 1 KiB block of a group: lane l
// takes row l / 8 of the group, position l % 8.  With this swizzle the 16-byte
// MFMA operand reads of 16 or 32 consecutive rows at one chunk, and the
// transposed reads of 4 consecutive rows x 32 B, hit distinct LDS banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz8(int r8) {
  return ((r8 >> 2) & 1) | (r8 & 2) | (((r8 ^ (r8 >> 1) ^ (r8 >> 2)) & 1) << 2);
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

// Remap so that every XCD receives chunks of c consecutive logical block ids, the XCDs taking
// the chunks in turn (XCD x: chunks x, x + 8, ..): neighbouring work items still share an L2,
// while work that grows or shrinks along the ids is spread evenly over the XCDs.  Each XCD
// walks its chunks in order; a last partial round of 8 c ids keeps the identity.
__device__ __forceinline__ int xcd_chunked_block(int b, int nblocks, int c) {
  const int full = (nblocks / (8 * c)) * (8 * c);
  if (b >= full) return b;
  const int x = b % 8, k = b / 8;
  return ((k / c) * 8 + x) * c + (k % c);
}

// The values of lanes l and l ^ 32 (or l ^ 16), as a pair (own half first or second does not
// matter to the symmetric reductions below).  v_permlane32_swap / v_permlane16_swap are
// VALU operations: no LDS round trip, unlike a general lane shuffle.
struct LanePair { float a, b; };
__device__ __forceinline__ LanePair pair_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor32(float v) { const LanePair p = pair_xor32(v); return fmaxf(p.a, p.b); }
__device__ __forceinline__ float sum_xor32(float v) { const LanePair p = pair_xor32(v); return p.a + p.b; }

// Inclusive prefix sum of v over the wave's lanes, and the wave's total (uniform), by DPP
// row shifts inside each 16-lane row (a source lane outside the row contributes 0) and the
// four row totals read from lanes 15, 31, 47 and 63: no LDS round trip.
__device__ __forceinline__ int wave_incl_scan(int v, int& total) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const int sh = d == 1 ? __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false)
                 : d == 2 ? __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false)
                 : d == 4 ? __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false)
                          : __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:d
    v += sh;
  }
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  total = r0 + r1 + r2 + r3;
  const int row = (int)(threadIdx.x & 63) >> 4;
  return v + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
}

// First token and token count of group grp of 128-row attention: G consecutive tokens
// from grp * G, or the entry of a batch's group table [NG, 2] (clamped into [0, T)).
__device__ __forceinline__ int2 group_span(const int32_t* ginfo, int grp, int G, int T) {
  if (ginfo == nullptr) return int2{grp * G, min(G, T - grp * G)};
  const int t0 = min(max(ginfo[2 * grp], 0), T);
  const int n = min(max(ginfo[2 * grp + 1], 0), min(G, T - t0));
  return int2{t0, n};
}

// max / sum over the 4 lanes l, l^16, l^32, l^48 (the 4 row groups of a 16x16 C tile)
__device__ __forceinline__ float max_over_rowgroups(float v) {
  const LanePair p = pair_xor16(v);
  return max_xor32(fmaxf(p.a, p.b));
}
__device__ __forceinline__ float sum_over_rowgroups(float v) {
  const LanePair p = pair_xor16(v);
  return sum_xor32(p.a + p.b);
}

}  // namespace dsa
