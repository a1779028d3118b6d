// Per-token sparse MQA prefill over the 576-wide bf16 latent.
//
// Definition ("[Perf][GLM-5.3-Flash] Dense/masked-MHA sparse prefill for the
// NoPE (256, 0, 256) layout ...", Purpose section; "[Perf][DSA] Grouped sparse
// prefill ...", commit message): every query token attends, for each of its H
// heads, over the latent rows of its own top-k selection; scores use all 576
// dims, values are the first 512 dims of the same rows; the result is
// out [T, H, 512] (bf16) and LSE [T, H] (fp32, natural log).  The pages find
// this kernel bound by the KV gather (2048 rows x 1152 B per token).
//
// MI355X design (one workgroup of 4 waves per (token, 16-head block)):
//  * the token's top-k row is read 64 entries at a time; wave 0 compacts the
//    valid entries (0 <= x < S, x <= position) with ballot/mbcnt;
//  * the 64 selected rows (72 x 16 B chunks each) are gathered with coalesced
//    16-byte loads into an LDS tile whose row stride is padded to 1168 B
//    (consecutive rows start 4 banks apart: conflict-free 16-byte reads);
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims read
//    from LDS, B = the 16 heads' query chunk held in registers;  each of the 4
//    waves computes the same 64 x 16 scores, so the softmax state is
//    wave-local and no cross-wave exchange is needed;
//  * O^T = V^T P^T, the waves splitting the 512 value columns (128 each).  The
//    probabilities go straight from the C registers of S^T into the B operand
//    (a consistent relabelling of the 32 keys of each MFMA step), V^T comes
//    from the LDS tile column-wise;
//  * fp32 online softmax in base 2 (scale folded with log2 e); l sums the
//    bf16-rounded probabilities that the MFMA actually multiplies.
//  * token order is reversed (long causal rows first) and block ids are
//    remapped so each XCD runs a contiguous token range: neighbouring tokens,
//    which share most of their rows, then hit the same L2.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kChunks = kDqk * 2 / 16;       // 72 chunks of 16 B per latent row
constexpr int kRowBytes = kDqk * 2 + 16;     // padded LDS row stride
constexpr int kRowHalves = kRowBytes / 2;
constexpr int kPtKeys = 64;
constexpr int kPtThreads = 256;

__global__ __launch_bounds__(kPtThreads) void pertoken_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, int64_t ld, int T, int H, int S, int cols,
    int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t tile[kPtKeys * kRowBytes];
  __shared__ int32_t kidx[kPtKeys];
  __shared__ int nvalid_s;

  const int nb = H >> 4;
  const int item = xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int tq = item / nb;
  const int token = T - 1 - tq;
  const int hb = item - tq * nb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;
  const int64_t pos = q_pos_offset + token;

  // B operand of S^T = K Q^T: head n of this block, dims 32 s + 8 g .. + 8
  bf16x8 qreg[kDqk / 32];
  {
    const uint16_t* qrow = q + ((size_t)token * H + hb * 16 + n) * kDqk + 8 * g;
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* tile16 = reinterpret_cast<const uint16_t*>(tile);
  const int32_t* trow = topk + (size_t)token * ld;

  for (int c0 = 0; c0 < cols; c0 += kPtKeys) {
    __syncthreads();  // previous tile consumed
    if (wave == 0) {
      const int c = c0 + lane;
      const int32_t x = c < cols ? trow[c] : -1;
      const bool v = x >= 0 && x < S && (int64_t)x <= pos;
      const uint64_t mk = ballot(v);
      if (v) kidx[lanes_below(mk)] = x;
      if (lane == 0) nvalid_s = __popcll(mk);
    }
    __syncthreads();
    const int nv = nvalid_s;
    if (nv == 0) continue;

    // gather the nv selected rows; rows nv..63 are zero-filled
#pragma unroll
    for (int it = 0; it < kPtKeys * kChunks / kPtThreads; ++it) {
      const int e = tid + it * kPtThreads;
      const int r = e / kChunks;
      const int ch = e - r * kChunks;
      uint4 val = {0u, 0u, 0u, 0u};
      if (r < nv) val = *reinterpret_cast<const uint4*>(kv + (size_t)kidx[r] * kDqk + ch * 8);
      *reinterpret_cast<uint4*>(tile + r * kRowBytes + ch * 16) = val;
    }
    __syncthreads();

    // scores of 64 keys (4 blocks of 16) for the 16 heads
    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = tile + (16 * kb + n) * kRowBytes + 16 * g;
#pragma unroll
      for (int s = 0; s < kDqk / 32; ++s)
        acc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(krow + 64 * s), qreg[s], acc);
      sacc[kb] = acc;  // acc[j] = score(key 16 kb + 4 g + j, head n)
    }

    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = (16 * kb + 4 * g + j < nv) ? sacc[kb][j] * scale_log2 : kNegInf;
        sacc[kb][j] = v;
        mt = fmaxf(mt, v);
      }
    mt = max_over_rowgroups(mt);
    const float m_new = fmaxf(m_run, mt);  // finite: the tile holds >= 1 valid key
    const float alpha = fast_exp2(m_run - m_new);
    float ls = 0.f;
    uint16_t pb[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t b = f32_to_bf16_bits(fast_exp2(sacc[kb][j] - m_new));
        pb[kb][j] = b;
        ls += bf16_bits_to_f32(b);
      }
    ls = sum_over_rowgroups(ls);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) o[cb] *= alpha;

    // O^T[cols of this wave] += V^T P^T; MFMA step ks covers keys 32 ks .. +32 with
    // k-slot (g, i) <-> key 32 ks + 16 (i / 4) + 4 g + (i % 4)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u16x8 pv = {pb[2 * ks][0], pb[2 * ks][1], pb[2 * ks][2], pb[2 * ks][3],
                        pb[2 * ks + 1][0], pb[2 * ks + 1][1], pb[2 * ks + 1][2], pb[2 * ks + 1][3]};
      const bf16x8 bop = __builtin_bit_cast(bf16x8, pv);
      const uint16_t* vbase = tile16 + (32 * ks + 4 * g) * kRowHalves + 128 * wave + n;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const uint16_t* vp = vbase + 16 * cb;
        const u16x8 a = {vp[0], vp[kRowHalves], vp[2 * kRowHalves], vp[3 * kRowHalves],
                         vp[16 * kRowHalves], vp[17 * kRowHalves], vp[18 * kRowHalves],
                         vp[19 * kRowHalves]};
        o[cb] = mfma16x16x32(__builtin_bit_cast(bf16x8, a), bop, o[cb]);
      }
    }
  }

  // o[cb][j] = O^T[col 128 wave + 16 cb + 4 g + j][head n]
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* orow = out + ((size_t)token * H + hb * 16 + n) * kDv + 128 * wave + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const u16x4 w = {f32_to_bf16_bits(o[cb][0] * inv), f32_to_bf16_bits(o[cb][1] * inv),
                     f32_to_bf16_bits(o[cb][2] * inv), f32_to_bf16_bits(o[cb][3] * inv)};
    *reinterpret_cast<u16x4*>(orow + 16 * cb) = w;
  }
  if (wave == 0 && g == 0)
    lse[(size_t)token * H + hb * 16 + n] =
        l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
}

hipError_t launch_pertoken_attn(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                float scale, uint16_t* out, float* lse, hipStream_t stream) {
  const long long items = (long long)T * (H / 16);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(pertoken_attn_kernel, dim3((unsigned)items), dim3(kPtThreads), 0, stream, q,
                     kv, topk, ld, T, H, S, cols, q_pos_offset, scale * kLog2e, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
