// Union list + per-token membership mask of a token group, and the bit-packed
// top-k mask of the masked-MHA routing.
//
// Group union ("[Perf][DSA] Grouped sparse prefill with the FlashMLA
// head-group-mask kernel", commit message and "How" section): for each group of
// G consecutive tokens, the ascending list of every position some member
// selects, -1 padded, its length, and one byte per list slot whose bit i says
// whether token gG + i selects that position.
//
// MI355X design: one workgroup per group.  A byte per KV position lives in LDS
// (a 32 KiB window of positions per pass); member i ORs bit i into the byte of
// each position it selects (LDS atomics commute, so the result does not depend
// on their order).  Each byte is then both "in the union" (non-zero) and the
// mask byte itself.  Compaction is ordered: every wave counts the non-zero
// bytes of its contiguous segment with ballot/popcount, the four counts are
// scanned, and a second pass writes each non-zero position at
// base + mbcnt(ballot) -- coalesced stores of consecutive slots.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kUnionThreads = 256;
constexpr int kUnionWaves = kUnionThreads / 64;
constexpr int kUnionWindow = 32768;  // positions per LDS pass (one byte each)

__global__ __launch_bounds__(kUnionThreads) void build_union_kernel(
    const int32_t* __restrict__ topk, int64_t ld, int T, int cols, int S, int64_t q_pos_offset,
    int G, int union_pad, int32_t* __restrict__ union_idx, int32_t* __restrict__ union_len,
    uint8_t* __restrict__ head_group_mask) {
  __shared__ uint32_t bytemap[kUnionWindow / 4];
  __shared__ int wave_count[kUnionWaves];

  const int NG = (T + G - 1) / G;
  const int g = NG - 1 - (int)blockIdx.x;  // later groups scan more positions: start them first
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = g * G;
  const int ntok = min(G, T - t0);

  // positions a member can select: [0, pend)
  int64_t pmax = q_pos_offset + t0 + ntok - 1;
  if (pmax > (int64_t)S - 1) pmax = (int64_t)S - 1;
  const int pend = pmax < 0 ? 0 : (int)(pmax + 1);

  int32_t* uout = union_idx + (size_t)g * union_pad;
  uint8_t* mout = head_group_mask + (size_t)g * union_pad;
  const uint8_t* bm = reinterpret_cast<const uint8_t*>(bytemap);

  int total = 0;
  for (int w0 = 0; w0 < pend; w0 += kUnionWindow) {
    const int wlen = min(kUnionWindow, pend - w0);
    for (int i = tid; i < (wlen + 3) / 4; i += kUnionThreads) bytemap[i] = 0u;
    __syncthreads();

    for (int e = tid; e < ntok * cols; e += kUnionThreads) {
      const int i = e / cols;
      const int c = e - i * cols;
      const int t = t0 + i;
      const int32_t x = topk[(size_t)t * ld + c];
      // selection rule: 0 <= x < S and x <= position of token t; x >= w0 >= 0 covers x >= 0
      if (x >= w0 && x - w0 < wlen && (int64_t)x <= q_pos_offset + t) {
        const int p = x - w0;
        atomicOr(&bytemap[p >> 2], (1u << i) << (8 * (p & 3)));
      }
    }
    __syncthreads();

    // ordered compaction: wave w owns positions [s0, s1) of this window
    const int seg = ((wlen + 64 * kUnionWaves - 1) / (64 * kUnionWaves)) * 64;
    const int s0 = wave * seg;
    const int s1 = min(wlen, s0 + seg);
    int cnt = 0;
    for (int p = s0; p < s1; p += 64) {
      const int pp = p + lane;
      cnt += __popcll(ballot(pp < s1 && bm[pp] != 0));
    }
    if (lane == 0) wave_count[wave] = cnt;
    __syncthreads();
    int base = total, wtotal = 0;
    for (int w = 0; w < kUnionWaves; ++w) {
      if (w < wave) base += wave_count[w];
      wtotal += wave_count[w];
    }
    for (int p = s0; p < s1; p += 64) {
      const int pp = p + lane;
      const uint8_t b = pp < s1 ? bm[pp] : (uint8_t)0;
      const uint64_t m = ballot(b != 0);
      if (b != 0) {
        const int o = base + lanes_below(m);
        if (o < union_pad) {  // always true when union_pad >= G * cols (checked on the host)
          uout[o] = w0 + pp;
          mout[o] = b;
        }
      }
      base += __popcll(m);
    }
    total += wtotal;
    __syncthreads();  // the next window reuses bytemap and wave_count
  }

  if (total > union_pad) total = union_pad;
  for (int j = total + tid; j < union_pad; j += kUnionThreads) {
    uout[j] = -1;
    mout[j] = 0;
  }
  if (tid == 0) union_len[g] = total;
}

// Bit-packed top-k membership for masked MHA ("[2/N][Attention] Enable masked MHA
// for sparse MLA prefills": the top-k mask buffer is zeroed and filled in a
// kernel).  bits[t][x / 32] bit (x % 32) = 1 iff x in sel(t).  One workgroup
// per token row; the row's words are built in LDS and written out coalesced,
// so every word (including the zero ones) is overwritten by each call.
constexpr int kBitsThreads = 256;
constexpr int kBitsWindowWords = 8192;  // 32 KiB of LDS: 262144 positions per pass

__global__ __launch_bounds__(kBitsThreads) void scatter_topk_bits_kernel(
    const int32_t* __restrict__ topk, int64_t ld, int T, int cols, int S, int64_t q_pos_offset,
    uint32_t* __restrict__ bits, int words) {
  __shared__ uint32_t row[kBitsWindowWords];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t pos = q_pos_offset + t;
  const int32_t* trow = topk + (size_t)t * ld;
  uint32_t* brow = bits + (size_t)t * words;
  for (int wb = 0; wb < words; wb += kBitsWindowWords) {
    const int nw = min(kBitsWindowWords, words - wb);
    for (int i = tid; i < nw; i += kBitsThreads) row[i] = 0u;
    __syncthreads();
    const int64_t lo = (int64_t)wb * 32, hi = lo + (int64_t)nw * 32;
    for (int c = tid; c < cols; c += kBitsThreads) {
      const int32_t x = trow[c];
      if (x >= 0 && x < S && (int64_t)x <= pos && x >= lo && x < hi) {
        const int p = (int)(x - lo);
        atomicOr(&row[p >> 5], 1u << (p & 31));
      }
    }
    __syncthreads();
    for (int i = tid; i < nw; i += kBitsThreads) brow[wb + i] = row[i];
    __syncthreads();
  }
}

hipError_t launch_build_union(const int32_t* topk, int64_t ld, int T, int cols, int S,
                              int64_t q_pos_offset, int G, int union_pad, int32_t* union_idx,
                              int32_t* union_len, uint8_t* head_group_mask, hipStream_t stream) {
  const int NG = (T + G - 1) / G;
  if (NG == 0) return hipSuccess;
  hipLaunchKernelGGL(build_union_kernel, dim3(NG), dim3(kUnionThreads), 0, stream, topk, ld, T,
                     cols, S, q_pos_offset, G, union_pad, union_idx, union_len, head_group_mask);
  return hipGetLastError();
}

hipError_t launch_scatter_topk_bits(const int32_t* topk, int64_t ld, int T, int cols, int S,
                                    int64_t q_pos_offset, uint32_t* bits, int words,
                                    hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_topk_bits_kernel, dim3(T), dim3(kBitsThreads), 0, stream, topk, ld,
                     T, cols, S, q_pos_offset, bits, words);
  return hipGetLastError();
}

}  // namespace dsa
