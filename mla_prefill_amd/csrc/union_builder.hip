// Union list + per-token membership mask of a token group, and the bit-packed
// top-k mask of the masked-MHA routing.
//
// Group union ("[Perf][DSA] Grouped sparse prefill with the FlashMLA
// head-group-mask kernel", commit message and "How" section): for each group of
// G consecutive tokens, the ascending list of every position some member
// selects, -1 padded, its length, and one byte per list slot whose bit i says
// whether token gG + i selects that position.
//
// Batches of requests over a paged KV cache ("[Perf][DSA] Grouped sparse prefill
// ...", "How" section: groups are consecutive tokens of one request, and the
// union's request-local positions become physical rows through the request's
// index conversion): groups are numbered request by request, each covers up to G
// consecutive tokens of one request, the union is built over request-local
// positions exactly as above, and each list entry is written as its physical row
// (block_table[r][x / page_size] * page_size + x % page_size).  Positions whose
// row falls outside the cache (or past the request's page table) are not
// selected.  The group table (first token, token count) is written alongside.
//
// MI355X design: one workgroup per group.  A byte per KV position lives in LDS
// (a 32 KiB window of positions per pass); member i ORs bit i into the byte of
// each position it selects (LDS atomics commute, so the result does not depend
// on their order).  Each byte is then both "in the union" (non-zero) and the
// mask byte itself.  Compaction is ordered: every wave counts the non-zero
// bytes of its contiguous segment, 16 bytes per lane per read, the four counts
// are scanned, and a second pass writes each non-zero position at base + its
// rank, consecutive slots in order (a sparse segment from each lane's prefix of
// the lanes' counts, a dense one 64 positions at a time by ballot ranks).
#include "common.h"
#include "kernels.h"

namespace dsa {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnionThreads = 256;
constexpr int kUnionWaves = kUnionThreads / 64;
constexpr int kUnionWindow = 32768;  // positions per LDS pass (one byte each)

// A batch of requests (device arrays; data contents are never errors, every index
// is checked before use).
struct ReqBatch {
  int R;
  const int32_t* cu_seqlens;   // [R + 1]: query tokens of request r are cu[r] .. cu[r + 1] - 1
  const int32_t* kv_lens;      // [R]: positions 0 .. kv_len - 1 exist
  const int32_t* q_pos_start;  // [R]: position of the request's first query token
  const int32_t* block_table;  // [R, bt_ld]: physical page of each request page
  int64_t bt_ld;
  int page_size;
  int num_slots;               // rows of the cache
};

// request of token t: the first r with cu[r + 1] > t (empty requests are skipped)
__device__ __forceinline__ int request_of(const ReqBatch& b, int t) {
  int lo = 0, hi = b.R - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (b.cu_seqlens[mid + 1] <= t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// physical row of request r's position x, or -1 (past the page table or the cache)
__device__ __forceinline__ int64_t physical_row(const ReqBatch& b, int r, int x) {
  const int pg = x / b.page_size;
  if ((int64_t)pg >= b.bt_ld) return -1;
  const int32_t page = b.block_table[(int64_t)r * b.bt_ld + pg];
  if (page < 0) return -1;
  const int64_t row = (int64_t)page * b.page_size + (x - pg * b.page_size);
  return row < b.num_slots ? row : -1;
}

// kVarlen = false: one sequence (group g = tokens gG ..), positions q_pos_offset + t,
// rows = positions.  kVarlen = true: the batch `b` (S, q_pos_offset unused).
template <bool kVarlen>
__global__ __launch_bounds__(kUnionThreads) void build_union_kernel(
    const int32_t* __restrict__ topk, int64_t ld, int T, int cols, int S, int64_t q_pos_offset,
    int G, int union_pad, int32_t* __restrict__ union_idx, int32_t* __restrict__ union_len,
    uint8_t* __restrict__ head_group_mask, ReqBatch b, int32_t* __restrict__ group_info) {
  __shared__ __align__(16) uint32_t bytemap[kUnionWindow / 4];
  __shared__ int wave_count[kUnionWaves];
  __shared__ int grp_req, grp_k, scan_tmp[kUnionThreads];

  const int NG = (int)gridDim.x;
  const int g = NG - 1 - (int)blockIdx.x;  // later groups scan more positions: start them first
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int t0, ntok, r = 0;
  int64_t pos0;  // position of the group's first token
  int S_eff;     // positions that exist
  if (!kVarlen) {
    t0 = g * G;
    ntok = min(G, T - t0);
    pos0 = q_pos_offset + t0;
    S_eff = S;
  } else {
    // group g is group k of request r: a block-wide scan of ceil(n_r / G) over the requests
    if (tid == 0) { grp_req = -1; grp_k = 0; }
    __syncthreads();
    int base = 0;
    for (int r0 = 0; r0 < b.R; r0 += kUnionThreads) {
      const int rr = r0 + tid;
      int n = 0;
      if (rr < b.R) n = max(0, min(b.cu_seqlens[rr + 1], T) - max(b.cu_seqlens[rr], 0));
      const int cnt = (n + G - 1) / G;
      scan_tmp[tid] = cnt;
      __syncthreads();
      for (int d = 1; d < kUnionThreads; d <<= 1) {  // inclusive scan (Hillis-Steele)
        const int v = tid >= d ? scan_tmp[tid - d] : 0;
        __syncthreads();
        scan_tmp[tid] += v;
        __syncthreads();
      }
      const int incl = base + scan_tmp[tid];
      if (rr < b.R && cnt > 0 && g >= incl - cnt && g < incl) { grp_req = rr; grp_k = g - (incl - cnt); }
      base += scan_tmp[kUnionThreads - 1];
      __syncthreads();
    }
    r = grp_req;
    if (r < 0) {  // past the batch's last group
      t0 = 0;
      ntok = 0;
      pos0 = 0;
      S_eff = 0;
    } else {
      const int c0 = max(b.cu_seqlens[r], 0);
      t0 = c0 + grp_k * G;
      ntok = min(G, min(b.cu_seqlens[r + 1], T) - t0);
      pos0 = (int64_t)b.q_pos_start[r] + (t0 - b.cu_seqlens[r]);
      S_eff = b.kv_lens[r];
    }
    if (tid == 0) {
      group_info[2 * g] = t0;
      group_info[2 * g + 1] = ntok;
    }
  }

  // positions a member can select: [0, pend)
  int64_t pmax = pos0 + ntok - 1;
  if (pmax > (int64_t)S_eff - 1) pmax = (int64_t)S_eff - 1;
  const int pend = (pmax < 0 || ntok <= 0) ? 0 : (int)(pmax + 1);

  int32_t* uout = union_idx + (size_t)g * union_pad;
  uint8_t* mout = head_group_mask + (size_t)g * union_pad;
  const uint8_t* bm = reinterpret_cast<const uint8_t*>(bytemap);

  int total = 0;
  for (int w0 = 0; w0 < pend; w0 += kUnionWindow) {
    const int wlen = min(kUnionWindow, pend - w0);
    for (int i = tid; i < (wlen + 3) / 4; i += kUnionThreads) bytemap[i] = 0u;
    __syncthreads();

    // (eight independent loads per thread before their LDS updates: one memory latency per
    // eight entries instead of one per entry)
    const int nent = ntok * cols;
    // rows of whole 16-byte vectors (the usual top-k widths): each thread loads 16 vectors
    // (64 entries) back to back -- unconditionally, at a clamped index, so that no load waits
    // under a branch -- and a group's 8 x 2048 entries arrive in one memory round trip
    const bool vec = !kVarlen && (cols & 3) == 0 && (ld & 3) == 0 && ((uintptr_t)topk & 15) == 0;
    const int nvec = vec ? nent >> 2 : 0;
    for (int v0 = tid; v0 < nvec; v0 += 16 * kUnionThreads) {
      i32x4 xs[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = 4 * min(v0 + u * kUnionThreads, nvec - 1);
        const int i = e / cols;
        xs[u] = *reinterpret_cast<const i32x4*>(topk + (size_t)(t0 + i) * ld + (e - i * cols));
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int v = v0 + u * kUnionThreads;
        const int i = (4 * v) / cols;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int32_t x = xs[u][c];
          if (v < nvec && x >= w0 && x - w0 < wlen && (int64_t)x <= pos0 + i) {
            const int p = x - w0;
            atomicOr(&bytemap[p >> 2], (1u << i) << (8 * (p & 3)));
          }
        }
      }
    }
    for (int e0 = vec ? nent : tid; e0 < nent; e0 += 8 * kUnionThreads) {
      int32_t xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kUnionThreads;
        xs[u] = -1;
        if (e < nent) {
          const int i = e / cols;
          xs[u] = topk[(size_t)(t0 + i) * ld + (e - i * cols)];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kUnionThreads;
        const int i = e / cols;
        const int32_t x = xs[u];
        // selection rule: 0 <= x < S and x <= position of token t; x >= w0 >= 0 covers x >= 0
        // (a batch also drops positions without a physical row); entries past the group
        // hold -1
        if (x >= w0 && x - w0 < wlen && (int64_t)x <= pos0 + i && (!kVarlen || physical_row(b, r, x) >= 0)) {
          const int p = x - w0;
          atomicOr(&bytemap[p >> 2], (1u << i) << (8 * (p & 3)));
        }
      }
    }
    __syncthreads();

    // ordered compaction: wave w owns positions [s0, s1) of this window.  A lane counts the
    // non-zero bytes of 16 at a time; the four wave totals are scanned; then a sparse segment
    // goes 1024 positions at a time (the lanes' counts scanned, each lane writing its entries
    // in order from base + its exclusive prefix) and a dense one 64 positions at a time
    // (ballot ranks, one slot per lane)
    const int seg = ((wlen + 1024 * kUnionWaves - 1) / (1024 * kUnionWaves)) * 1024;
    const int s0 = wave * seg;
    const int s1 = min(wlen, s0 + seg);
    // bit k: byte p + k of the map is non-zero (p % 16 == 0; bytes at or past wlen count as zero)
    auto nonzero16 = [&](int p, uint4& w) -> uint32_t {
      w = *reinterpret_cast<const uint4*>(bm + p);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t m = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hi = (((ws[j] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | ws[j]) & 0x80808080u;  // bit 8 i + 7: byte i
        m |= (((hi >> 7) * 0x00204081u) >> 21 & 0xfu) << (4 * j);                         // gathered to bits 0..3
      }
      const int valid = wlen - p;
      return valid >= 16 ? m : (m & ((1u << valid) - 1u));
    };
    int cnt = 0;
    for (int p = s0 + 16 * lane; p < s1; p += 1024) {
      uint4 w;
      cnt += __popc(nonzero16(p, w));
    }
    int wsum;
    (void)wave_incl_scan(cnt, wsum);
    if (lane == 0) wave_count[wave] = wsum;
    __syncthreads();
    int base = total, wtotal = 0;
    for (int w = 0; w < kUnionWaves; ++w) {
      if (w < wave) base += wave_count[w];
      wtotal += wave_count[w];
    }
    if (4 * wsum > s1 - s0) {
      // a dense segment (more than one position in four): 64 consecutive positions per step,
      // one slot per lane (coalesced stores)
      for (int q = s0; q < s1; q += 64) {
        const int pp = q + lane;
        const uint8_t mb = pp < s1 ? bm[pp] : (uint8_t)0;
        const uint64_t bal = ballot(mb != 0);
        if (mb != 0) {
          const int o = base + lanes_below(bal);
          if (o < union_pad) {  // always true when union_pad >= G * cols (checked on the host)
            uout[o] = kVarlen ? (int32_t)physical_row(b, r, w0 + pp) : w0 + pp;
            mout[o] = mb;
          }
        }
        base += __popcll(bal);
      }
    } else {
      for (int c0 = s0; c0 < s1; c0 += 1024) {
        const int p = c0 + 16 * lane;
        uint4 w = {0u, 0u, 0u, 0u};
        uint32_t m = p < s1 ? nonzero16(p, w) : 0u;
        const int c = __popc(m);
        int n;
        int o = base + wave_incl_scan(c, n) - c;
        while (m != 0u) {
          const int k = __ffs(m) - 1;
          if (o < union_pad) {
            const uint32_t wk = (k & 8) ? ((k & 4) ? w.w : w.z) : ((k & 4) ? w.y : w.x);
            uout[o] = kVarlen ? (int32_t)physical_row(b, r, w0 + p + k) : w0 + p + k;
            mout[o] = (uint8_t)(wk >> (8 * (k & 3)));
          }
          ++o;
          m &= m - 1u;
        }
        base += n;
      }
    }
    total += wtotal;
    __syncthreads();  // the next window reuses bytemap and wave_count
  }

  if (total > union_pad) total = union_pad;
  // padding up to a whole number of 64-slot blocks only: readers stop at the tile holding the
  // last entry, and the rest of the row (most of it for compact unions) is not written
  const int pad_end = min(union_pad, (total + 63) & ~63);
  for (int j = total + tid; j < pad_end; j += kUnionThreads) {
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
constexpr int kBitsWindowWords = 4096;  // 16 KiB of LDS: 131072 positions per pass

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
    // (eight independent loads per thread before their LDS updates: one memory latency per
    // eight entries instead of one per entry)
    for (int c0 = tid; c0 < cols; c0 += 8 * kBitsThreads) {
      int32_t xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * kBitsThreads;
        xs[u] = c < cols ? trow[c] : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int32_t x = xs[u];
        if (x >= 0 && x < S && (int64_t)x <= pos && x >= lo && x < hi) {
          const int p = (int)(x - lo);
          atomicOr(&row[p >> 5], 1u << (p & 31));
        }
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
  hipLaunchKernelGGL(build_union_kernel<false>, dim3(NG), dim3(kUnionThreads), 0, stream, topk, ld, T,
                     cols, S, q_pos_offset, G, union_pad, union_idx, union_len, head_group_mask,
                     ReqBatch{}, (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_build_union_varlen(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                     const int32_t* cu_seqlens, const int32_t* kv_lens,
                                     const int32_t* q_pos_start, const int32_t* block_table,
                                     int64_t bt_ld, int page_size, int num_slots, int G, int max_groups,
                                     int union_pad, int32_t* group_info, int32_t* union_idx,
                                     int32_t* union_len, uint8_t* head_group_mask, hipStream_t stream) {
  if (max_groups == 0) return hipSuccess;
  const ReqBatch b{R, cu_seqlens, kv_lens, q_pos_start, block_table, bt_ld, page_size, num_slots};
  hipLaunchKernelGGL(build_union_kernel<true>, dim3(max_groups), dim3(kUnionThreads), 0, stream, topk,
                     ld, T, cols, 0, (int64_t)0, G, union_pad, union_idx, union_len, head_group_mask, b,
                     group_info);
  return hipGetLastError();
}

// Request-local top-k entries as physical rows ("[Perf][DSA] Grouped sparse prefill ...",
// "How" section: the index conversion to physical rows), -1 where the entry selects
// nothing (negative, past the request's KV, beyond the token's position, or without a
// physical row).  One workgroup per token.
__global__ __launch_bounds__(256) void convert_req_index_kernel(const int32_t* __restrict__ topk,
                                                                 int64_t ld, int T, int cols, ReqBatch b,
                                                                 int32_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int r = request_of(b, t);
  const int64_t pos = (int64_t)b.q_pos_start[r] + (t - b.cu_seqlens[r]);
  const int kvl = b.kv_lens[r];
  const int32_t* trow = topk + (size_t)t * ld;
  int32_t* orow = out + (size_t)t * cols;
  for (int c = threadIdx.x; c < cols; c += 256) {
    const int32_t x = trow[c];
    int32_t row = -1;
    if (x >= 0 && x < kvl && (int64_t)x <= pos) row = (int32_t)physical_row(b, r, x);
    orow[c] = row;
  }
}

hipError_t launch_convert_req_index(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                    const int32_t* cu_seqlens, const int32_t* kv_lens,
                                    const int32_t* q_pos_start, const int32_t* block_table, int64_t bt_ld,
                                    int page_size, int num_slots, int32_t* out, hipStream_t stream) {
  if (T == 0 || cols == 0) return hipSuccess;
  const ReqBatch b{R, cu_seqlens, kv_lens, q_pos_start, block_table, bt_ld, page_size, num_slots};
  hipLaunchKernelGGL(convert_req_index_kernel, dim3(T), dim3(256), 0, stream, topk, ld, T, cols, b, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Routing by the union's size.  The grouped form costs about one 128-row tile per 32 union
// slots of a group; the per-token form about rho(H) such tiles per 32 selections of a
// token.  With the union built, one workgroup sums ceil(union_len / 32) over the groups and
// writes route[0] = 1 (skip the grouped kernels) when the sum exceeds `limit` (the per-token
// cost in the same tiles), else route[1] = 1 (skip the per-token kernel); route[2] = the
// union tiles (saturated at 2^31 - 1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_by_union_kernel(const int32_t* __restrict__ union_len, int NG,
                                                             int union_pad, double limit, int32_t* route) {
  __shared__ long long part[256];
  long long s = 0;
  for (int g = threadIdx.x; g < NG; g += 256) {
    const int u = min(max(union_len[g], 0), union_pad);
    s += (u + 31) / 32;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long tiles = part[0];
    const bool grouped = (double)tiles <= limit;
    route[0] = grouped ? 0 : 1;
    route[1] = grouped ? 1 : 0;
    route[2] = (int32_t)min(tiles, (long long)INT32_MAX);
  }
}

hipError_t launch_route_by_union(const int32_t* union_len, int NG, int union_pad, double limit, int32_t* route,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(route_by_union_kernel, dim3(1), dim3(256), 0, stream, union_len, NG, union_pad, limit, route);
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
