// 128-row sparse attention over a per-workgroup key list: the grouped routing.
//
// Definition ("[Perf][DSA] Grouped sparse prefill with the FlashMLA
// head-group-mask kernel", commit message and "How" section): G = 128 / H
// consecutive tokens are presented as 128 pseudo-heads (row r = i * H + h for
// token gG + i, head h) that attend over the sorted union of the group's top-k
// rows; the membership byte of each union slot restricts row r to the slots
// its own token selected (bit i), which reproduces per-token sparse attention
// exactly.  Rows of tokens >= T (partial last group) are neither loaded nor
// stored.
//
// The same kernel runs the per-token routing at H = 128 (G = 1): rows are the
// token's 128 heads and the key list is its top-k row, filtered by the
// selection rule (0 <= x < S, x <= position) instead of a membership byte.
//
// MI355X design (one workgroup of 8 waves per group, 2 waves per SIMD):
//  * per tile, 32 key slots are gathered (72 x 16 B chunks per row) into an
//    LDS tile with a 1168 B row stride;
//  * QK^T is split by rows: wave w owns rows 16 w .. 16 w + 15 (for H = 16 that
//    is exactly one token), holds their query in registers and computes
//    S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = keys from LDS);  masking
//    and the fp32 online softmax are applied in registers to its own rows;
//  * PV is split by value columns: wave w owns columns 64 w .. 64 w + 63 for
//    all 128 rows (O^T = V^T P^T, 8 x 4 accumulator tiles); the bf16
//    probabilities and the per-row rescale factors travel through LDS;
//  * the row's l sums the bf16-rounded probabilities the MFMA multiplies.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kGDqk = 576;
constexpr int kGDv = 512;
constexpr int kGChunks = kGDqk * 2 / 16;    // 72
constexpr int kGRowBytes = kGDqk * 2 + 16;  // 1168
constexpr int kGRowHalves = kGRowBytes / 2;
constexpr int kGKeys = 32;
constexpr int kGThreads = 512;
constexpr int kPStride = 40;  // halves per row of the probability buffer (32 + 8 pad)

template <bool kPerToken>
__global__ __launch_bounds__(kGThreads) void rows128_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ keys, int64_t keys_ld, const int32_t* __restrict__ union_len,
    const uint8_t* __restrict__ hgmask, int T, int H, int S, int ncols, int64_t q_pos_offset,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t tile[kGKeys * kGRowBytes];
  __shared__ __align__(16) uint16_t pbuf[128 * kPStride];
  __shared__ float alpha_s[128];
  __shared__ float linv_s[128];
  __shared__ int32_t kidx[kGKeys];
  __shared__ uint8_t kmask[kGKeys];

  const int G = 128 / H;
  const int NG = (T + G - 1) / G;
  const int grp = NG - 1 - xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;
  const int t0 = grp * G;

  // the row this lane's wave owns for QK^T / softmax
  const int r_own = 16 * wave + n;
  const int i_own = r_own / H;
  const int h_own = r_own - i_own * H;
  const int tok_own = t0 + i_own;
  const bool row_live = tok_own < T;

  bf16x8 qreg[kGDqk / 32];
  if (row_live) {
    const uint16_t* qrow = q + ((size_t)tok_own * H + h_own) * kGDqk + 8 * g;
#pragma unroll
    for (int s = 0; s < kGDqk / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < kGDqk / 32; ++s) qreg[s] = bf16x8{};
  }

  int nkeys;
  if (kPerToken) {
    nkeys = ncols;
  } else {
    nkeys = union_len[grp];
    nkeys = nkeys < 0 ? 0 : (nkeys > ncols ? ncols : nkeys);
  }
  const int32_t* klist = keys + (size_t)grp * keys_ld;
  const uint8_t* mlist = kPerToken ? nullptr : hgmask + (size_t)grp * keys_ld;
  const int64_t pos = q_pos_offset + t0;  // per-token mode: the token's position

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[8][4];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) o[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* tile16 = reinterpret_cast<const uint16_t*>(tile);

  for (int j0 = 0; j0 < nkeys; j0 += kGKeys) {
    __syncthreads();  // previous tile and probabilities consumed
    if (tid < kGKeys) {
      const int j = j0 + tid;
      int32_t x = -1;
      uint8_t mb = 0;
      if (j < nkeys) {
        x = klist[j];
        const bool in_range = x >= 0 && x < S;
        if (kPerToken)
          mb = (in_range && (int64_t)x <= pos) ? (uint8_t)1 : (uint8_t)0;
        else
          mb = in_range ? mlist[j] : (uint8_t)0;
        if (mb == 0) x = -1;
      }
      kidx[tid] = x;
      kmask[tid] = mb;
    }
    __syncthreads();

    for (int e = tid; e < kGKeys * kGChunks; e += kGThreads) {
      const int r = e / kGChunks;
      const int ch = e - r * kGChunks;
      const int32_t x = kidx[r];
      uint4 val = {0u, 0u, 0u, 0u};
      if (x >= 0) val = *reinterpret_cast<const uint4*>(kv + (size_t)x * kGDqk + ch * 8);
      *reinterpret_cast<uint4*>(tile + r * kGRowBytes + ch * 16) = val;
    }
    __syncthreads();

    // scores for this wave's 16 rows over the 32 slots
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = tile + (16 * kb + n) * kGRowBytes + 16 * g;
#pragma unroll
      for (int s = 0; s < kGDqk / 32; ++s)
        acc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(krow + 64 * s), qreg[s], acc);
      sacc[kb] = acc;  // acc[j] = score(slot 16 kb + 4 g + j, row r_own)
    }

    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int slot = 16 * kb + 4 * g + j;
        const bool ok = ((kmask[slot] >> i_own) & 1) != 0;
        const float v = ok ? sacc[kb][j] * scale_log2 : kNegInf;
        sacc[kb][j] = v;
        mt = fmaxf(mt, v);
      }
    mt = max_over_rowgroups(mt);
    const float m_new = fmaxf(m_run, mt);
    const bool any = m_new != kNegInf;  // this row has met an allowed slot
    const float alpha = any ? fast_exp2(m_run - m_new) : 1.f;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u16x4 pw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t b = any ? f32_to_bf16_bits(fast_exp2(sacc[kb][j] - m_new)) : (uint16_t)0;
        pw[j] = b;
        ls += bf16_bits_to_f32(b);
      }
      *reinterpret_cast<u16x4*>(pbuf + r_own * kPStride + 16 * kb + 4 * g) = pw;
    }
    ls = sum_over_rowgroups(ls);
    l_run = l_run * alpha + ls;
    m_run = m_new;
    if (g == 0) alpha_s[r_own] = alpha;
    __syncthreads();

    // O^T[64 w .. 64 w + 63][all rows] += V^T P^T over the 32 slots
    bf16x8 va[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint16_t* vp = tile16 + (8 * g) * kGRowHalves + 64 * wave + 16 * cb + n;
      const u16x8 a = {vp[0], vp[kGRowHalves], vp[2 * kGRowHalves], vp[3 * kGRowHalves],
                       vp[4 * kGRowHalves], vp[5 * kGRowHalves], vp[6 * kGRowHalves],
                       vp[7 * kGRowHalves]};
      va[cb] = __builtin_bit_cast(bf16x8, a);
    }
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      const float al = alpha_s[16 * rb + n];
      const bf16x8 pop = *reinterpret_cast<const bf16x8*>(pbuf + (16 * rb + n) * kPStride + 8 * g);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) o[rb][cb] = mfma16x16x32(va[cb], pop, o[rb][cb] * al);
    }
  }

  if (g == 0) {
    linv_s[r_own] = l_run > 0.f ? 1.f / l_run : 0.f;
    if (row_live)
      lse[(size_t)tok_own * H + h_own] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
  }
  __syncthreads();

  // o[rb][cb][j] = O^T[col 64 w + 16 cb + 4 g + j][row 16 rb + n]
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    const int row = 16 * rb + n;
    const int i = row / H;
    const int h = row - i * H;
    const int tok = t0 + i;
    if (tok >= T) continue;
    const float inv = linv_s[row];
    uint16_t* orow = out + ((size_t)tok * H + h) * kGDv + 64 * wave + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const u16x4 w = {f32_to_bf16_bits(o[rb][cb][0] * inv), f32_to_bf16_bits(o[rb][cb][1] * inv),
                       f32_to_bf16_bits(o[rb][cb][2] * inv), f32_to_bf16_bits(o[rb][cb][3] * inv)};
      *reinterpret_cast<u16x4*>(orow + 16 * cb) = w;
    }
  }
}

hipError_t launch_grouped_attn(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                               const int32_t* union_len, const uint8_t* head_group_mask, int T,
                               int H, int S, int union_pad, float scale, uint16_t* out, float* lse,
                               hipStream_t stream) {
  const int G = 128 / H;
  const int NG = (T + G - 1) / G;
  if (NG == 0) return hipSuccess;
  hipLaunchKernelGGL(rows128_attn_kernel<false>, dim3(NG), dim3(kGThreads), 0, stream, q, kv,
                     union_idx, (int64_t)union_pad, union_len, head_group_mask, T, H, S, union_pad,
                     (int64_t)0, scale * kLog2e, out, lse);
  return hipGetLastError();
}

hipError_t launch_pertoken_rows128(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                   int64_t ld, int T, int S, int cols, int64_t q_pos_offset,
                                   float scale, uint16_t* out, float* lse, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rows128_attn_kernel<true>, dim3(T), dim3(kGThreads), 0, stream, q, kv, topk,
                     ld, (const int32_t*)nullptr, (const uint8_t*)nullptr, T, 128, S, cols,
                     q_pos_offset, scale * kLog2e, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
