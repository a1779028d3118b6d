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
// MI355X design (one workgroup of 8 waves per (256-query tile, head); 2 waves
// per SIMD):
//  * each wave owns 32 query rows; their 256-dim queries sit in registers as
//    the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, the full-rate
//    shape on gfx950);
//  * 32-key tiles of K and V (512 B per key row of one head) and the matching
//    mask words stream through a 3-stage LDS ring by asynchronous global->LDS
//    DMA, two tiles ahead of the compute; one barrier per tile;
//  * rows are stored with a per-row chunk rotation (mrot below): the 16-byte
//    K reads (16 rows, one column) and the transposed V reads (4 rows x 32 B)
//    are both free of bank conflicts, and every copy instruction fills two
//    whole rows;
//  * causal test and top-k bit are applied to the S^T accumulators in
//    registers; fp32 online softmax in base 2; the bf16 probabilities go
//    straight from the accumulators into the B operand of O^T = V^T P^T (keys
//    relabelled consistently), V^T comes from ds_read_b64_tr_b16;
//  * key tiles past the causal diagonal of the tile's last query are never
//    visited; query tiles run longest first.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kMD = 256;                              // qk and v head dim
constexpr int kMWaves = 8;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMQ = 32 * kMWaves;                     // query rows per workgroup
constexpr int kMKeys = 32;                            // keys per tile
constexpr int kMStages = 3;
constexpr int kMRowBytes = kMD * 2;                   // 512 B rows, 32 chunks of 16 B
constexpr int kMTileBytes = kMKeys * kMRowBytes;      // K (or V) tile
constexpr int kMStageBytes = 2 * kMTileBytes;
constexpr int kMDmaTotal = kMStageBytes / 1024;       // 32 wave copies per tile (2 rows each)
constexpr int kMDmaPerWave = kMDmaTotal / kMWaves;    // 4
constexpr int kMOpsPerTile = kMDmaPerWave + 1;        // + the mask-word copy
static_assert(kMDmaTotal % kMWaves == 0, "copies must split evenly over the waves");

// Chunk c of tile row r is stored at chunk position (c - rot(r)) mod 32 of the
// row.  With rot(r) = 2 r + r / 8, the 16-byte reads of one chunk by 16
// consecutive rows hit 16 distinct positions, and the transposed reads of two
// neighbouring chunks by 4 consecutive rows (a 4-aligned group) hit 8 distinct
// positions: no LDS bank conflicts for either operand.
__device__ __forceinline__ int mrot(int r) { return (2 * r + (r >> 3)) & 31; }

__global__ __launch_bounds__(kMThreads) void masked_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint32_t* __restrict__ bits, int words, int T, int S,
    int H, int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t stage[kMStages][kMStageBytes];
  __shared__ __align__(16) uint32_t maskw[kMStages][kMWaves][64];

  const int nqt = (T + kMQ - 1) / kMQ;
  const int lb = xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int qt = nqt - 1 - lb / H;
  const int h = lb - (lb / H) * H;
  const int q0 = qt * kMQ;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hi = lane >> 5, m = lane & 31;
  const int row = q0 + 32 * wave + m;  // query token of this lane's row
  const bool live = row < T;
  // last key this row may see (positions beyond S - 1 cannot be selected); -1 for rows >= T
  int64_t rpos64 = q_pos_offset + row;
  if (rpos64 > S - 1) rpos64 = S - 1;
  const int rpos = live ? (int)rpos64 : -1;

  bf16x8 qreg[kMD / 16];
  if (live) {
    const uint16_t* qrow = q + ((size_t)row * H + h) * kMD + 8 * hi;
#pragma unroll
    for (int s = 0; s < kMD / 16; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < kMD / 16; ++s) qreg[s] = bf16x8{};
  }
  // complete the query loads now, before any asynchronous copy is in flight
#pragma unroll
  for (int s = 0; s < kMD / 16; ++s) asm volatile("" : : "v"(qreg[s]));

  const int last = min(T, q0 + kMQ) - 1;
  int64_t kend64 = q_pos_offset + last + 1;
  if (kend64 > S) kend64 = S;
  const int kend = (int)kend64;
  const int ntiles = (kend + kMKeys - 1) / kMKeys;
  const int mrow = min(row, T - 1);

  auto issue = [&](int t) {
    const int k0 = t * kMKeys;
    uint8_t* st = stage[t % kMStages];
#pragma unroll
    for (int u = 0; u < kMDmaPerWave; ++u) {
      const int i = wave + kMWaves * u;          // copy i: rows 2 i, 2 i + 1 of the K|V stage
      const int which = i >= kMDmaTotal / 2 ? 1 : 0;
      const int r = 2 * (i - which * (kMDmaTotal / 2)) + hi;
      const int c = (m + mrot(r)) & 31;          // lane m of the row fills position m
      int key = k0 + r;
      key = key < kend ? key : kend - 1;
      dma16((which ? v : k) + ((size_t)key * H + h) * kMD + c * 8, lds_addr(st + 1024 * i));
    }
    dma4(bits + (size_t)mrow * words + (k0 >> 5), lds_addr(&maskw[t % kMStages][wave][0]));
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[kMD / 32];
#pragma unroll
  for (int cb = 0; cb < kMD / 32; ++cb) o[cb] = f32x16{};

  const int g16 = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (s16 >> 2);         // transposed-read row within a 16-key step
  const int vchunk = 2 * (g16 & 1) + ((s16 & 3) >> 1);  // chunk within a 32-column block
  const int vhalf = 8 * (s16 & 1);                      // byte offset within the chunk
  const int krot = hi - mrot(m);                        // K read: position of chunk 2 s + hi

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles)
      wait_vmcnt<kMOpsPerTile>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // tile t visible to all waves; stage (t + 2) % 3 free
    if (t + 2 < ntiles) issue(t + 2);

    const uint8_t* kt = stage[t % kMStages];
    const uint8_t* vt = kt + kMTileBytes;
    const int k0 = t * kMKeys;

    f32x16 sacc = {};
    const uint8_t* kp = kt + m * kMRowBytes;
    const int kr = loop_local(krot);
#pragma unroll
    for (int s0 = 0; s0 < kMD / 16; s0 += 2) {
      bf16x8 ka[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        ka[u] = *reinterpret_cast<const bf16x8*>(kp + 16 * ((2 * (s0 + u) + kr) & 31));
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc = mfma32x32x16(ka[u], qreg[s0 + u], sacc);
      sched_fence();
    }
    // sacc[j] = score(key k0 + 8 (j / 4) + 4 hi + j % 4, row)

    // bits of this lane's 16 keys: key 8 (j / 4) + 4 hi + j % 4 -> bit 8 (j / 4) + j % 4 of mw
    const uint32_t mw = maskw[t % kMStages][wave][m] >> (4 * hi);
    const int lim = rpos - k0 - 4 * hi;  // key offset 8 (j / 4) + j % 4 must be <= lim
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kk = 8 * (j >> 2) + (j & 3);
      const bool ok = ((mw >> kk) & 1u) != 0u && kk <= lim;
      const float val = ok ? sacc[j] * scale_log2 : kNegInf;
      sacc[j] = val;
      mt = fmaxf(mt, val);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const bool any = m_new != kNegInf;
    const float alpha = any ? fast_exp2(m_run - m_new) : 1.f;
    uint16_t pb[16];
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      pb[j] = any ? f32_to_bf16_bits(fast_exp2(sacc[j] - m_new)) : (uint16_t)0;
      ls += bf16_bits_to_f32(pb[j]);
    }
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < kMD / 32; ++cb) o[cb] *= alpha;

    // O^T += V^T P^T: step st covers keys 16 st .. 16 st + 15 with k-slot (hi, i) <->
    // key 16 st + 8 (i / 4) + 4 hi + i % 4, i.e. accumulator registers 8 st .. 8 st + 7
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u16x8 pv = {pb[8 * st + 0], pb[8 * st + 1], pb[8 * st + 2], pb[8 * st + 3],
                        pb[8 * st + 4], pb[8 * st + 5], pb[8 * st + 6], pb[8 * st + 7]};
      const bf16x8 bop = __builtin_bit_cast(bf16x8, pv);
      const int r0 = 16 * st + vrow, r1 = r0 + 8;
      const uint8_t* v0 = vt + r0 * kMRowBytes + vhalf;
      const uint8_t* v1 = vt + r1 * kMRowBytes + vhalf;
      const int p0 = loop_local(vchunk - mrot(r0)), p1 = loop_local(vchunk - mrot(r1));
#pragma unroll
      for (int cb = 0; cb < kMD / 32; ++cb) {
        const u16x4 lo = lds_read_tr16(v0 + 16 * ((4 * cb + p0) & 31));
        const u16x4 up = lds_read_tr16(v1 + 16 * ((4 * cb + p1) & 31));
        const u16x8 a = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        o[cb] = mfma32x32x16(__builtin_bit_cast(bf16x8, a), bop, o[cb]);
        if (cb & 1) sched_fence();
      }
    }
  }

  if (!live) return;
  // o[cb][j] = O^T[col 32 cb + 8 (j / 4) + 4 hi + j % 4][row]
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* orow = out + ((size_t)row * H + h) * kMD + 4 * hi;
#pragma unroll
  for (int cb = 0; cb < kMD / 32; ++cb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u16x4 w = {f32_to_bf16_bits(o[cb][4 * jj + 0] * inv), f32_to_bf16_bits(o[cb][4 * jj + 1] * inv),
                       f32_to_bf16_bits(o[cb][4 * jj + 2] * inv), f32_to_bf16_bits(o[cb][4 * jj + 3] * inv)};
      *reinterpret_cast<u16x4*>(orow + 32 * cb + 8 * jj) = w;
    }
  if (hi == 0)
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
