// Masked dense MHA for sparse-MLA prefill, NoPE layout (qk 256 = nope 256 +
// rope 0, v 256).
//
// Definition ("[2/N][Attention] Enable masked MHA for sparse MLA prefills",
// Purpose section; "[Perf][GLM-5.3-Flash] Dense/masked-MHA sparse prefill for
// the NoPE (256, 0, 256) layout + skip the NoPE K concat", commit messages):
// below a length threshold, full-head attention over the up-projected per-head
// K and V with mask = causal AND top-k membership simulates DSA; with no rope
// part the key is k_nope itself, so no K concat is built -- this kernel reads
// k_nope in place.  Token t sits at position q_pos_offset + t (chunked
// context); the membership bits come from the bit-packed [T, ceil(S/32)] mask
// that scatter_topk_bits_kernel writes.
//
// MI355X design (one workgroup of 4 waves per (64-query tile, head)):
//  * each wave owns 16 query rows; their 256-dim queries sit in registers;
//  * 64-key tiles of K and V (512 B per key row of one head) are staged in
//    LDS with a padded 528 B stride; key tiles past the causal diagonal of the
//    tile's last query are never visited;
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16, then the causal test and the
//    top-k bit (two mask words per row and tile) are applied in registers;
//  * fp32 online softmax in base 2; P goes from the S^T accumulators straight
//    into the B operand of O^T = V^T P^T (keys relabelled consistently);
//  * query tiles run longest first (most causal key tiles).
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kMD = 256;                   // qk and v head dim
constexpr int kMRowBytes = kMD * 2 + 16;   // 528
constexpr int kMRowHalves = kMRowBytes / 2;
constexpr int kMQ = 64;                    // query rows per workgroup
constexpr int kMKeys = 64;                 // keys per tile
constexpr int kMThreads = 256;
constexpr int kMChunks = kMD * 2 / 16;     // 32 chunks of 16 B per key row

__global__ __launch_bounds__(kMThreads) void masked_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint32_t* __restrict__ bits, int words, int T, int S,
    int H, int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t ktile[kMKeys * kMRowBytes];
  __shared__ __align__(16) uint8_t vtile[kMKeys * kMRowBytes];

  const int nqt = (T + kMQ - 1) / kMQ;
  const int lb = xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int qt = nqt - 1 - lb / H;
  const int h = lb - (lb / H) * H;
  const int q0 = qt * kMQ;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;

  const int row = q0 + 16 * wave + n;  // query token of this lane's row
  const bool live = row < T;
  const int64_t rpos = q_pos_offset + row;

  bf16x8 qreg[kMD / 32];
  if (live) {
    const uint16_t* qrow = q + ((size_t)row * H + h) * kMD + 8 * g;
#pragma unroll
    for (int s = 0; s < kMD / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < kMD / 32; ++s) qreg[s] = bf16x8{};
  }

  // keys the tile can see: [0, kend)
  const int last = min(T, q0 + kMQ) - 1;
  int64_t kend64 = q_pos_offset + last + 1;
  if (kend64 > S) kend64 = S;
  const int kend = (int)kend64;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vtile);
  const uint32_t* brow = bits + (size_t)(live ? row : 0) * words;

  for (int k0 = 0; k0 < kend; k0 += kMKeys) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kMKeys * kMChunks / kMThreads; ++it) {
      const int e = tid + it * kMThreads;
      const int r = e / kMChunks;
      const int ch = e - r * kMChunks;
      const int key = k0 + r;
      uint4 kval = {0u, 0u, 0u, 0u}, vval = {0u, 0u, 0u, 0u};
      if (key < kend) {
        const size_t off = ((size_t)key * H + h) * kMD + ch * 8;
        kval = *reinterpret_cast<const uint4*>(k + off);
        vval = *reinterpret_cast<const uint4*>(v + off);
      }
      *reinterpret_cast<uint4*>(ktile + r * kMRowBytes + ch * 16) = kval;
      *reinterpret_cast<uint4*>(vtile + r * kMRowBytes + ch * 16) = vval;
    }
    // top-k bits of this row for keys k0 .. k0 + 63
    const int w0 = k0 >> 5;
    const uint32_t mw0 = (live && w0 < words) ? brow[w0] : 0u;
    const uint32_t mw1 = (live && w0 + 1 < words) ? brow[w0 + 1] : 0u;
    __syncthreads();

    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = ktile + (16 * kb + n) * kMRowBytes + 16 * g;
#pragma unroll
      for (int s = 0; s < kMD / 32; ++s)
        acc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(krow + 64 * s), qreg[s], acc);
      sacc[kb] = acc;  // acc[j] = score(key k0 + 16 kb + 4 g + j, row)
    }

    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = 16 * kb + 4 * g + j;
        const uint32_t word = kk < 32 ? mw0 : mw1;
        const bool ok = ((word >> (kk & 31)) & 1u) != 0u && (int64_t)(k0 + kk) <= rpos &&
                        k0 + kk < kend;
        const float val = ok ? sacc[kb][j] * scale_log2 : kNegInf;
        sacc[kb][j] = val;
        mt = fmaxf(mt, val);
      }
    mt = max_over_rowgroups(mt);
    const float m_new = fmaxf(m_run, mt);
    const bool any = m_new != kNegInf;
    const float alpha = any ? fast_exp2(m_run - m_new) : 1.f;
    float ls = 0.f;
    uint16_t pb[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t b = any ? f32_to_bf16_bits(fast_exp2(sacc[kb][j] - m_new)) : (uint16_t)0;
        pb[kb][j] = b;
        ls += bf16_bits_to_f32(b);
      }
    ls = sum_over_rowgroups(ls);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] *= alpha;

#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u16x8 pv = {pb[2 * ks][0], pb[2 * ks][1], pb[2 * ks][2], pb[2 * ks][3],
                        pb[2 * ks + 1][0], pb[2 * ks + 1][1], pb[2 * ks + 1][2], pb[2 * ks + 1][3]};
      const bf16x8 bop = __builtin_bit_cast(bf16x8, pv);
      const uint16_t* vbase = vt16 + (32 * ks + 4 * g) * kMRowHalves + n;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        const uint16_t* vp = vbase + 16 * cb;
        const u16x8 a = {vp[0], vp[kMRowHalves], vp[2 * kMRowHalves], vp[3 * kMRowHalves],
                         vp[16 * kMRowHalves], vp[17 * kMRowHalves], vp[18 * kMRowHalves],
                         vp[19 * kMRowHalves]};
        o[cb] = mfma16x16x32(__builtin_bit_cast(bf16x8, a), bop, o[cb]);
      }
    }
  }

  if (!live) return;
  // o[cb][j] = O^T[col 16 cb + 4 g + j][row]
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* orow = out + ((size_t)row * H + h) * kMD + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    const u16x4 w = {f32_to_bf16_bits(o[cb][0] * inv), f32_to_bf16_bits(o[cb][1] * inv),
                     f32_to_bf16_bits(o[cb][2] * inv), f32_to_bf16_bits(o[cb][3] * inv)};
    *reinterpret_cast<u16x4*>(orow + 16 * cb) = w;
  }
  if (g == 0)
    lse[(size_t)row * H + h] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
}

hipError_t launch_masked_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* v,
                             const uint32_t* bits, int words, int T, int S, int H,
                             int64_t q_pos_offset, float scale, uint16_t* out, float* lse,
                             hipStream_t stream) {
  const long long blocks = (long long)((T + kMQ - 1) / kMQ) * H;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(masked_mha_kernel, dim3((unsigned)blocks), dim3(kMThreads), 0, stream, q,
                     k_nope, v, bits, words, T, S, H, q_pos_offset, scale * kLog2e, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
