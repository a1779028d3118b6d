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
// MI355X design: one wave per (token, 16-head block), one wave per workgroup so
// that four of them share a CU's LDS and run independently (no barriers):
//  * the token's top-k row is consumed 16 entries at a time; the entries are
//    wave-uniform and come through scalar loads; invalid entries (-1, out of
//    range, beyond the token's position) are masked, steps with no valid
//    entry are skipped;
//  * the 16 rows of a step (72 x 16 B chunks each) are copied global -> LDS by
//    asynchronous DMA into a 2-stage ring, one step ahead of the compute; LDS
//    rows are padded to 1168 B (292 dwords, 36 mod 64 banks), which makes both
//    the 16-byte K reads (16 rows, one column) and the transposed V reads
//    (4 rows x 32 B) free of bank conflicts;
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = the 16
//    heads' queries in registers); the probabilities leave the accumulators
//    directly as the B operand of O^T = V^T P^T (v_mfma_f32_16x16x16_bf16),
//    V^T comes from one ds_read_b64_tr_b16 per operand;
//  * fp32 online softmax in base 2 with lazy rescaling (O and l are rescaled
//    only when a head's max grows by more than 2^8);
//  * token order is reversed (long causal rows first) and block ids are
//    remapped so each XCD runs a contiguous token range: neighbouring tokens,
//    which share most of their rows, then hit the same L2.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kPKeys = 16;                     // keys per pipeline step
constexpr int kPRowBytes = kDqk * 2 + 16;      // 1168: 72 data chunks + 1 pad chunk
constexpr int kPSlots = kPRowBytes / 16;       // 73
constexpr int kPDma = (kPKeys * kPSlots + 63) / 64;  // 19 wave copies per step
constexpr int kPStageBytes = kPDma * 1024;     // the tail of the last copy lands in slack
constexpr int kPStages = 2;
constexpr float kPSlack = 8.f;                 // lazy-rescale threshold (log2 units)

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(s16x4_t a, s16x4_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(64) void pertoken_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, int64_t ld, int T, int H, int S, int cols,
    int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t stage[kPStages][kPStageBytes];

  const int nb = H >> 4;
  const int item = xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int tq = item / nb;
  const int token = T - 1 - tq;
  const int hb = item - tq * nb;
  const int lane = threadIdx.x;
  const int g = lane >> 4, n = lane & 15;
  int64_t pos64 = q_pos_offset + token;
  if (pos64 > S - 1) pos64 = S - 1;  // positions beyond S - 1 cannot be selected
  const int pos = uniform((int)pos64);

  // B operand of S^T = K Q^T: head n of this block, dims 32 s + 8 g .. + 8
  bf16x8 qreg[kDqk / 32];
  {
    const uint16_t* qrow = q + ((size_t)token * H + hb * 16 + n) * kDqk + 8 * g;
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s) asm volatile("" : : "v"(qreg[s]));  // loads done before any copy
  }

  const int32_t* trow = topk + (size_t)token * ld;
  const int nsteps = (cols + kPKeys - 1) / kPKeys;

  // entries of step j (wave-uniform, scalar loads) and their validity bits
  auto entries = [&](int j, int32_t (&e)[kPKeys]) -> uint32_t {
    const_i32* tp = uniform_const(trow + kPKeys * j);
    const int avail = cols - kPKeys * j;
    uint32_t vbits = 0;
#pragma unroll
    for (int r = 0; r < kPKeys; ++r) {
      const int32_t x = r < avail ? tp[r] : -1;
      const bool ok = x >= 0 && x <= pos;  // pos <= S - 1
      e[r] = ok ? x : 0;
      vbits |= ok ? (1u << r) : 0u;
    }
    return vbits;
  };

  // copy the 16 rows e[0..15] into stage st: copy i fills slots 64 i .. 64 i + 63,
  // slot s = row s / 73, chunk s % 73 (chunk 72 is padding and gets chunk 0)
  auto issue = [&](const int32_t (&e)[kPKeys], int st) {
#pragma unroll
    for (int i = 0; i < kPDma; ++i) {
      const int r0 = (64 * i) / kPSlots;                  // first row this copy touches
      const int thr = kPSlots * (r0 + 1) - 64 * i;        // lanes >= thr are in row r0 + 1
      const bool up = lane >= thr;
      const int r = up ? r0 + 1 : r0;
      const int c = 64 * i + lane - kPSlots * r;
      int32_t x = up ? e[r0 + 1 < kPKeys ? r0 + 1 : r0] : e[r0];
      if (r >= kPKeys) x = 0;                             // slack beyond the last row
      dma16(kv + (size_t)x * kDqk + (c < 72 ? c : 0) * 8, lds_addr(stage[st] + 1024 * i));
    }
  };

  float m_run = kNegInf, l_run = 0.f;  // per head n (replicated over the 4 lane groups)
  f32x4 o[kDv / 16];
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int koff = n * kPRowBytes + 16 * g;                          // K: row n, chunk 4 s + g
  const int voff = (4 * g + (lane & 15) / 4) * kPRowBytes + 8 * (lane & 3);  // V^T: see below

  int32_t ecur[kPKeys], enxt[kPKeys];
  int j = 0;
  uint32_t vcur = 0;
  while (j < nsteps && (vcur = entries(j, ecur)) == 0u) ++j;
  if (j < nsteps) issue(ecur, 0);
  int st = 0;
  while (j < nsteps) {
    int jn = j + 1;
    uint32_t vnxt = 0;
    while (jn < nsteps && (vnxt = entries(jn, enxt)) == 0u) ++jn;
    int tofs = st * kPStageBytes;  // this step's stage, usable only after its copies landed
    if (jn < nsteps) {
      issue(enxt, st ^ 1);
      tofs = wait_vmcnt_dep<kPDma>(tofs);
    } else {
      tofs = wait_vmcnt_dep<0>(tofs);
    }

    const uint8_t* tile = &stage[0][0] + tofs;
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s)
      sacc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(tile + koff + 64 * s), qreg[s], sacc);
    // sacc[jj] = score(key 4 g + jj of the step, head n)

    float mt = kNegInf;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float val = ((vcur >> (4 * g + jj)) & 1u) ? sacc[jj] * scale_log2 : kNegInf;
      sacc[jj] = val;
      mt = fmaxf(mt, val);
    }
    mt = max_over_rowgroups(mt);
    const bool need = mt > m_run + kPSlack;
    if (ballot(need) != 0) {
      const float m_new = need ? mt : m_run;
      const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < kDv / 16; ++cb) o[cb] *= alpha;
      m_run = m_new;
    }
    const float msafe = m_run == kNegInf ? 0.f : m_run;
    float ls = 0.f;
    bf16x4 pb;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float p = fast_exp2(sacc[jj] - msafe);
      ls += p;
      pb[jj] = (__bf16)p;
    }
    l_run += sum_over_rowgroups(ls);
    const s16x4_t bop = __builtin_bit_cast(s16x4_t, pb);  // P^T[keys 4 g + jj][head n]

    // O^T[col 16 cb + 4 g + jj][head n] += V^T P^T.  A operand: lane (g, n) needs
    // V[key 4 g + jj][col 16 cb + n]; the transposed read gives it when lane
    // (g, s) of a 16-lane group addresses row 4 g + s / 4, columns 16 cb + 4 (s % 4).
#pragma unroll
    for (int cb = 0; cb < kDv / 16; ++cb) {
      const u16x4 a = lds_read_tr16(tile + voff + 32 * cb);
      o[cb] = mfma16x16x16(__builtin_bit_cast(s16x4_t, a), bop, o[cb]);
    }

    vcur = vnxt;
#pragma unroll
    for (int r = 0; r < kPKeys; ++r) ecur[r] = enxt[r];
    j = jn;
    st ^= 1;
  }

  // o[cb][jj] = O^T[col 16 cb + 4 g + jj][head n]
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* orow = out + ((size_t)token * H + hb * 16 + n) * kDv + 4 * g;
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) {
    const bf16x4 w = {(__bf16)(o[cb][0] * inv), (__bf16)(o[cb][1] * inv), (__bf16)(o[cb][2] * inv),
                      (__bf16)(o[cb][3] * inv)};
    *reinterpret_cast<bf16x4*>(orow + 16 * cb) = w;
  }
  if (g == 0)
    lse[(size_t)token * H + hb * 16 + n] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
}

hipError_t launch_pertoken_attn(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                float scale, uint16_t* out, float* lse, hipStream_t stream) {
  const long long items = (long long)T * (H / 16);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(pertoken_attn_kernel, dim3((unsigned)items), dim3(64), 0, stream, q, kv, topk,
                     ld, T, H, S, cols, q_pos_offset, scale * kLog2e, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
