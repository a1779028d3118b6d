// FP8 KV latent: decode of the codes to bf16, once per latent row.
//
// The pages gate quantized KV caches off the grouped path ("[Perf][DSA] Grouped
// sparse prefill ...", "How" section) and define no FP8 format.  The format
// here: OCP E4M3 codes (gfx950's native FP8) with a float32 scale, one per row
// or one for the whole cache; element (x, i) = e4m3(kv8[x, i]) * scale.
//
// MI355X design: every E4M3 value is exactly a bf16 number (3 mantissa bits,
// exponents 2^-9 .. 2^8), so the codes are decoded to bf16 with no rounding
// and the scale is NOT applied here: the attention kernels multiply each key's
// raw score by its row's scale and each probability by it before the PV
// product, so the result is attention over the exact values e4m3 * scale.
// The attention kernels take their latent rows from L2 (a 16k-token chunk
// gathers ~37 GB of rows of which ~1.7 GB pass L2), and each row is gathered
// about T * k / S times (2048 at T = S = 16k); decoding inside the gather would
// redo the conversion at every use, while this pass decodes each row once into
// a caller workspace: 1 byte read and 2 written per element.
//  * decode_fp8_kernel: one thread per 16 codes (one 16-byte load, two 16-byte
//    stores), v_cvt_pk_f32_fp8 for the decode;
//  * decode_paged_fp8_kernel: a batch over a paged cache: the pages a request
//    can reach (positions < kv_len) are decoded into a compact workspace,
//    request after request, with each workspace row's scale and a block table
//    over the workspace.
#include "common.h"
#include "kernels.h"

namespace dsa {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 16 codes -> 16 bf16 bit patterns (two 16-byte words), exact
__device__ __forceinline__ void decode16(uint4 c, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // bytes 0, 1 and 2, 3 of the word, in order; a float32 holding an E4M3 value has at most
    // 4 significant bits, so dropping its low 16 bits is exact
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    o[2 * i] = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
    o[2 * i + 1] = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
  }
  lo = uint4{o[0], o[1], o[2], o[3]};
  hi = uint4{o[4], o[5], o[6], o[7]};
}

__global__ __launch_bounds__(256) void decode_fp8_kernel(const uint8_t* __restrict__ kv8, int64_t nchunks,
                                                         uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  const uint4 c = *reinterpret_cast<const uint4*>(kv8 + 16 * i);
  uint4 lo, hi;
  decode16(c, lo, hi);
  uint4* o = reinterpret_cast<uint4*>(out + 16 * i);
  o[0] = lo;
  o[1] = hi;
}

// Workgroup (p, r): page p of request r (pages 0 .. ceil(kv_len / page_size) - 1 are
// reachable).  Request r's pages go to compact pages off(r) .. off(r) + n_r - 1, off(r) =
// the reachable pages of requests 0 .. r - 1.  The block table over the workspace gets
// off(r) + p for a reachable page whose source page id is valid and fits the workspace,
// and -1 otherwise (no position maps there); entries past a request's reachable pages
// get -1 too.  Each decoded row's scale goes to ws_scale (the single scale when the
// cache has one).
__global__ __launch_bounds__(256) void decode_paged_fp8_kernel(
    const uint8_t* __restrict__ cache8, const float* __restrict__ scale, int per_row, int num_pages,
    int d, const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ block_table,
    int64_t bt_ld, int page_size, int ws_pages, uint16_t* __restrict__ out_cache,
    float* __restrict__ out_scale, int32_t* __restrict__ out_bt) {
  const int r = (int)blockIdx.y;
  const int64_t p = blockIdx.x;  // p < bt_ld
  auto npages = [&](int rr) -> int64_t {
    const int64_t len = kv_lens[rr];
    return len > 0 ? (len + page_size - 1) / page_size : 0;
  };
  int64_t off = 0;
  for (int rr = 0; rr < r; ++rr) off += npages(rr);
  const int64_t n = npages(r);
  const bool reach = p < n;
  const int32_t src = reach ? block_table[(size_t)r * bt_ld + p] : -1;
  const bool ok = reach && src >= 0 && src < num_pages && off + p < ws_pages;
  if (threadIdx.x == 0) out_bt[(size_t)r * bt_ld + p] = ok ? (int32_t)(off + p) : -1;
  if (!ok) return;
  const int cpr = d / 16;  // 16-code chunks per row
  const int64_t nch = (int64_t)page_size * cpr;
  const uint8_t* sp = cache8 + (size_t)src * page_size * d;
  uint16_t* dp = out_cache + (size_t)(off + p) * page_size * d;
  for (int64_t i = threadIdx.x; i < nch; i += 256) {
    uint4 lo, hi;
    decode16(*reinterpret_cast<const uint4*>(sp + 16 * i), lo, hi);
    uint4* o = reinterpret_cast<uint4*>(dp + 16 * i);
    o[0] = lo;
    o[1] = hi;
  }
  for (int i = threadIdx.x; i < page_size; i += 256)
    out_scale[(off + p) * page_size + i] = scale[per_row ? (int64_t)src * page_size + i : 0];
}

hipError_t launch_decode_fp8(const uint8_t* kv8, int64_t rows, int d, uint16_t* out, hipStream_t stream) {
  const int64_t nchunks = rows * (d / 16);
  if (nchunks == 0) return hipSuccess;
  const int64_t blocks = (nchunks + 255) / 256;
  hipLaunchKernelGGL(decode_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv8, nchunks, out);
  return hipGetLastError();
}

hipError_t launch_decode_paged_fp8(const uint8_t* cache8, const float* scale, int per_row, int num_slots, int d,
                                   int R, const int32_t* kv_lens, const int32_t* block_table, int64_t bt_ld,
                                   int page_size, int ws_pages, uint16_t* out_cache, float* out_scale,
                                   int32_t* out_bt, hipStream_t stream) {
  if (R == 0 || bt_ld == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_paged_fp8_kernel, dim3((unsigned)bt_ld, (unsigned)R), dim3(256), 0, stream,
                     cache8, scale, per_row, num_slots / page_size, d, kv_lens, block_table, bt_ld,
                     page_size, ws_pages, out_cache, out_scale, out_bt);
  return hipGetLastError();
}

}  // namespace dsa
