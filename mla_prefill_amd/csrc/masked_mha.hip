// Masked dense MHA for sparse-MLA prefill, and its mask-free special case (dense
// causal MHA), for the per-head geometries (qk_nope, qk_rope, v) = (256, 0, 256),
// (192, 64, 256) and (128, 64, 128).
//
// Definition ("[2/N][Attention] Enable masked MHA for sparse MLA prefills",
// Purpose section; "[Perf][GLM-5.3-Flash] Dense/masked-MHA sparse prefill for
// the NoPE (256, 0, 256) layout + skip the NoPE K concat", commit messages and
// the masked-MHA allow-list of its description): below a length threshold,
// full-head attention over the up-projected per-head K and V with mask =
// causal AND top-k membership simulates DSA.  The key of a head is k_nope
// followed by the k_pe shared by all heads; with no rope part it is k_nope
// itself, and either way this kernel reads both in place (no K concat is
// built).  Token t sits at position q_pos_offset + t (chunked context); the
// membership bits come from the bit-packed [T, ceil(S/32)] mask that
// scatter_topk_bits_kernel writes.
//
// MI355X design (one workgroup of 8 waves per (256-query tile, head); 2 waves
// per SIMD):
//  * each wave owns 32 query rows; their queries (up to 12 k-steps in
//    registers, the rest in a lane-private LDS area) are the B operand of
//    S^T = K Q^T (v_mfma_f32_32x32x16_bf16, the full-rate shape on gfx950);
//  * 32-key tiles of K and V (one head's rows) and the matching mask words
//    stream through a 3-stage LDS ring by asynchronous global->LDS DMA, two
//    tiles ahead of the compute; one barrier per tile.  Each wave copy moves
//    128 B of 8 consecutive key rows into the swizzled 8-row-group layout
//    (common.h), so a lane's source address is its row plus an immediate, and
//    every operand read is a per-lane base plus an immediate with no LDS bank
//    conflicts;
//  * the causal test and the top-k bit select scores in registers (bit-field
//    insert of -inf); the running max is taken on raw scores and the softmax
//    scale is folded into one fused multiply-add before the base-2
//    exponential; O and l are rescaled only when a row's max grows by more
//    than 2^8; the bf16 probabilities go straight from the accumulators into
//    the B operand of O^T = V^T P^T (keys relabelled consistently), V^T comes
//    from ds_read_b64_tr_b16;
//  * key tiles past the causal diagonal of the tile's last query are never
//    visited; query tiles run longest first.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kMWaves = 8;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMQ = 32 * kMWaves;                     // query rows per workgroup
constexpr int kMKeys = 32;                            // keys per tile
constexpr int kMStages = 3;
constexpr float kRescaleSlack = 8.f;                  // rescale O only when the max grows by > 2^8
constexpr int kMQRegMax = 12;                         // query k-steps kept in registers (at most)

// Geometry (kDN, kDR, kDV): the key is k_nope (kDN dims, per head) followed by k_pe (kDR
// dims, shared by every head), the value kDV dims per head: (256, 0, 256) NoPE -- K is
// k_nope itself; (192, 64, 256); (128, 64, 128).
// kDense: plain causal attention (every causal key selected): no mask words are copied and
// tiles below the diagonal of all of a wave's rows skip the select.
template <int kDN, int kDR, int kDV, bool kDense>
__global__ __launch_bounds__(kMThreads) void masked_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kpe,
    const uint16_t* __restrict__ v, const uint32_t* __restrict__ bits, int words, int T, int S,
    int H, int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int kDQK = kDN + kDR;
  static_assert(kDN % 64 == 0 && kDR % 64 == 0 && kDV % 64 == 0, "whole 128-byte blocks per row");
  constexpr int kKBlocks = kDQK / 64, kVBlocks = kDV / 64;  // 1 KiB blocks per 8-row group
  constexpr int kKGroupBytes = 1024 * kKBlocks, kVGroupBytes = 1024 * kVBlocks;
  constexpr int kKTileBytes = 4 * kKGroupBytes;         // 32 keys of K
  constexpr int kStageBytes = kKTileBytes + 4 * kVGroupBytes;
  constexpr int kQSteps = kDQK / 16;                    // k-steps of S^T = K Q^T
  constexpr int kQRegSteps = kQSteps < kMQRegMax ? kQSteps : kMQRegMax;
  constexpr int kQLdsSteps = kQSteps - kQRegSteps;      // the rest sit in LDS (lane-private)
  constexpr int kCB = kDV / 32;                         // O^T column blocks
  // copies per wave per tile (K waves 0..3, V waves 4..7), + the mask-word copy
  constexpr int kOpsK = kKBlocks + (kDense ? 0 : 1), kOpsV = kVBlocks + (kDense ? 0 : 1);
  __shared__ __align__(16) uint8_t stage[kMStages][kStageBytes];
  __shared__ __align__(16) uint32_t maskw[kDense ? 1 : kMStages][kMWaves][64];
  __shared__ __align__(16) uint4 qlds[kMWaves][kQLdsSteps > 0 ? kQLdsSteps : 1][64];

  // longest query tiles first; consecutive blocks take consecutive heads, so the
  // round-robin XCD dispatch keeps each head on one XCD and balances the work
  const int nqt = (T + kMQ - 1) / kMQ;
  const int lb = (int)blockIdx.x;
  const int qt = nqt - 1 - lb / H;
  const int h = lb - (lb / H) * H;
  const int q0 = qt * kMQ;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;  // (wave: a scalar)
  const int hi = lane >> 5, m = lane & 31;
  const int row = q0 + 32 * wave + m;  // query token of this lane's row
  const bool live = row < T;
  // last key this row may see (positions beyond S - 1 cannot be selected); -1 for rows >= T
  int64_t rpos64 = q_pos_offset + row;
  if (rpos64 > S - 1) rpos64 = S - 1;
  const int rpos = live ? (int)rpos64 : -1;

  // queries; a negative scale is applied as |scale| on negated queries so that the
  // running max can be taken on raw scores
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sc = fabsf(scale_log2);
  // (steps kQRegSteps.. go to a lane-private LDS area: the registers are needed to keep
  // operand reads in flight)
  bf16x8 qreg[kQRegSteps];
  {
    const uint16_t* qrow = q + ((size_t)row * H + h) * kDQK + 8 * hi;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      uint4 w = {0u, 0u, 0u, 0u};
      if (live) w = *reinterpret_cast<const uint4*>(qrow + 16 * s);
      w.x ^= qsign; w.y ^= qsign; w.z ^= qsign; w.w ^= qsign;
      if (s < kQRegSteps)
        qreg[s] = __builtin_bit_cast(bf16x8, w);
      else
        qlds[wave][s - kQRegSteps][lane] = w;
    }
  }
  // complete the query loads now, before any asynchronous copy is in flight
#pragma unroll
  for (int s = 0; s < kQRegSteps; ++s) asm volatile("" : : "v"(qreg[s]));

  const int last = min(T, q0 + kMQ) - 1;
  int64_t kend64 = q_pos_offset + last + 1;
  if (kend64 > S) kend64 = S;
  const int kend = (int)kend64;
  const int ntiles = (kend + kMKeys - 1) / kMKeys;
  const int mrow = min(row, T - 1);

  // copies: wave w fills K (w < 4, kKBlocks blocks) or V (w >= 4, kVBlocks blocks) rows
  // 8 (w % 4) .. + 7; lane l takes row l / 8 of the group, position l % 8 (chunk 8 c + pos
  // ^ swizzle)
  const bool kwave = wave < 4;
  const int cgrp = wave & 3;
  const int crow = 8 * cgrp + (lane >> 3);
  const int cchunk = (lane & 7) ^ swz8(lane >> 3) ^ cgrp;
  // (K rows: blocks 0 .. kDN / 64 - 1 from k_nope, the rest from k_pe)
  const int kdim = kwave ? kDN : kDV;
  const uint16_t* cbase = (kwave ? k : v) + (size_t)h * kdim + 8 * cchunk;
  const size_t key_stride = (size_t)H * kdim;
  // k_pe element e of a row sits at dim kDN + e of the key row
  const uint16_t* pbase = kDR > 0 ? kpe + 8 * cchunk - kDN : cbase;
  const uint32_t cdst = kwave ? cgrp * kKGroupBytes : kKTileBytes + cgrp * kVGroupBytes;

  auto issue = [&](int t) {
    int key = t * kMKeys + crow;
    key = key < kend ? key : kend - 1;
    const uint16_t* src = cbase + (size_t)key * key_stride;
    const uint16_t* psrc = kDR > 0 ? pbase + (size_t)key * kDR : src;
    const uint32_t dst = lds_addr(stage[t % kMStages]) + cdst;
    // (the global address carries the block offset: an instruction offset would also
    // move the LDS destination of an LDS-DMA load)
    if (kwave) {
#pragma unroll
      for (int c = 0; c < kKBlocks; ++c) dma16((kDR > 0 && 64 * c >= kDN ? psrc : src) + 64 * c, dst + 1024 * c);
    } else {
#pragma unroll
      for (int c = 0; c < kVBlocks; ++c) dma16(src + 64 * c, dst + 1024 * c);
    }
    if constexpr (!kDense)
      dma4(bits + (size_t)mrow * words + ((t * kMKeys) >> 5), lds_addr(&maskw[t % kMStages][wave][0]));
  };

  float m_run = kNegInf, l_run = 0.f;  // m_run: reference max of the exponents (log2 units)
  f32x16 o[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) o[cb] = f32x16{};

  // K reads (A of S^T): row m, chunk 2 s + hi -> 4 bases, one per s % 4, plus (s / 4) KiB
  const int kx = swz8(m & 7) ^ (m >> 3) ^ hi;
  int kofs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kofs[u] = (m >> 3) * kKGroupBytes + (m & 7) * 128 + 16 * ((2 * u) ^ kx);
  // transposed V reads: row 16 st + 8 uu + 4 hi + s16 / 4, columns 32 cb + 16 (g16 % 2) + 4 (s16 % 4)
  const int g16 = lane >> 4, s16 = lane & 15;
  const int vr8 = 4 * hi + (s16 >> 2);
  const int vx = (2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ swz8(vr8);
  const int vbase = vr8 * 128 + 8 * (s16 & 1);

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 >= ntiles)
      wait_vmcnt<0>();
    else if (kwave)
      wait_vmcnt<kOpsK>();
    else
      wait_vmcnt<kOpsV>();
    __syncthreads();  // tile t visible to all waves; stage (t + 2) % 3 free
    if (t + 2 < ntiles) issue(t + 2);

    // one stage offset per iteration (kept opaque so no per-stage address sets are hoisted)
    const int sofs = loop_local((t % kMStages) * kStageBytes);
    const uint8_t* kt = &stage[0][0] + sofs;
    const uint8_t* vt = kt + kKTileBytes;
    const int k0 = t * kMKeys;

    // K operand reads run kMAhead steps ahead of the MFMAs (the order is pinned: left to
    // itself the scheduler puts every read right before its MFMA and waits out its latency)
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(&qlds[wave][0][0]) + loop_local(16 * lane);
    auto kread = [&](int s) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(kt + kofs[s & 3] + 1024 * (s >> 2));
    };
    auto qread = [&](int s) -> bf16x8 {
      return s < kQRegSteps ? qreg[s < kQRegSteps ? s : 0]
                            : *reinterpret_cast<const bf16x8*>(qb + 1024 * (s - kQRegSteps));
    };
    constexpr int kMAhead = 4;
    bf16x8 kw[kMAhead], qw[kMAhead];
#pragma unroll
    for (int s = 0; s < kMAhead; ++s) {
      kw[s] = kread(s);
      qw[s] = qread(s);
    }
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      sacc = mfma32x32x16(kw[s % kMAhead], qw[s % kMAhead], sacc);
      if (s + kMAhead < kQSteps) {
        kw[s % kMAhead] = kread(s + kMAhead);
        qw[s % kMAhead] = qread(s + kMAhead);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // sacc[j] = raw score(key k0 + 8 (j / 4) + 4 hi + j % 4, row)

    // allowed keys: top-k bit AND key <= position; bit kk <-> key k0 + 4 hi + kk
    const int lim = rpos - k0 - 4 * hi;
    const uint32_t causal = lim >= 31 ? 0xffffffffu : (lim < 0 ? 0u : ((2u << lim) - 1u));
    float mt = kNegInf;
    if (kDense && ballot(lim < 31) == 0) {
      // every key of the tile is causal for every row of the wave
#pragma unroll
      for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[j]);
    } else {
      uint32_t allowed = causal;
      if constexpr (!kDense)
        allowed &= *reinterpret_cast<const uint32_t*>(
                       reinterpret_cast<const uint8_t*>(&maskw[0][wave][m]) +
                       loop_local((t % kMStages) * (int)sizeof(maskw[0]))) >> (4 * hi);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kk = 8 * (j >> 2) + (j & 3);
        const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)allowed, kk, 1);  // all ones if allowed
        // (the element goes through a scalar first: a bit cast applied directly to a
        // vector element reads element 0 with this compiler)
        const float raw = sacc[j];
        const float val = __builtin_bit_cast(float, (sel & __builtin_bit_cast(uint32_t, raw)) |
                                                        (~sel & 0xff800000u));
        sacc[j] = val;
        mt = fmaxf(mt, val);
      }
    }
    mt = max_xor32(mt) * sc;
    // lazy rescale: move the reference max only when this tile exceeds it by > 2^8
    const bool need = mt > m_run + kRescaleSlack;
    if (ballot(need) != 0) {
      // rows that keep their max keep alpha = 1 (m_run may still be -inf there)
      const float alpha = need ? fast_exp2(m_run - mt) : 1.f;  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) o[cb] *= alpha;
      m_run = need ? mt : m_run;
    }
    const float nm = m_run == kNegInf ? 0.f : -m_run;
    float ls = 0.f;
    bf16x8 bop[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pj = fast_exp2(__builtin_fmaf(sacc[j], sc, nm));
      ls += pj;
      bop[j >> 3][j & 7] = (__bf16)pj;
    }
    l_run += ls;  // this half's keys; the halves are summed at the end

    // O^T += V^T P^T: step st covers keys 16 st .. 16 st + 15 with k-slot (hi, i) <->
    // key 16 st + 8 (i / 4) + 4 hi + i % 4, i.e. accumulator registers 8 st .. 8 st + 7
    // MFMA i (0 .. 2 kCB - 1) is step i / kCB, column block i % kCB; its V^T operand is read
    // kMVAhead MFMAs ahead (order pinned as for QK)
    auto vread = [&](int i) -> bf16x8 {
      const int st = i / kCB, cb = i % kCB;
      // rows 16 st + 8 uu + vr8 are in group 2 st + uu; chunk 4 cb + c2 is in block cb / 2
      const int p0 = 16 * (vx ^ (4 * (cb & 1)) ^ (2 * st));
      const int p1 = 16 * (vx ^ (4 * (cb & 1)) ^ (2 * st + 1));
      const u16x4 lo = lds_read_tr16(vt + (2 * st) * kVGroupBytes + 1024 * (cb >> 1) + vbase + p0);
      const u16x4 up = lds_read_tr16(vt + (2 * st + 1) * kVGroupBytes + 1024 * (cb >> 1) + vbase + p1);
      return __builtin_bit_cast(bf16x8, u16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    constexpr int kMVAhead = 3;
    bf16x8 vw[kMVAhead];
#pragma unroll
    for (int i = 0; i < kMVAhead; ++i) vw[i] = vread(i);
#pragma unroll
    for (int i = 0; i < 2 * kCB; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      o[i % kCB] = mfma32x32x16(vw[i % kMVAhead], bop[i / kCB], o[i % kCB]);
      if (i + kMVAhead < 2 * kCB) vw[i % kMVAhead] = vread(i + kMVAhead);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  const float l_tot = sum_xor32(l_run);  // (before the exit: every lane takes part)
  if (!live) return;
  // o[cb][j] = O^T[col 32 cb + 8 (j / 4) + 4 hi + j % 4][row]
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* orow = out + ((size_t)row * H + h) * kDV + 4 * hi;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bf16x4 w = {(__bf16)(o[cb][4 * jj + 0] * inv), (__bf16)(o[cb][4 * jj + 1] * inv),
                        (__bf16)(o[cb][4 * jj + 2] * inv), (__bf16)(o[cb][4 * jj + 3] * inv)};
      *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * jj) = w;
    }
  if (hi == 0)
    lse[(size_t)row * H + h] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
}

template <int kDN, int kDR, int kDV>
static void launch_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                       const uint16_t* v, const uint32_t* bits, int words, int T, int S, int H,
                       int64_t q_pos_offset, float scale, uint16_t* out, float* lse, hipStream_t stream) {
  const long long blocks = (long long)((T + kMQ - 1) / kMQ) * H;
  // no membership bits: every causal key is selected (plain causal attention)
  if (bits == nullptr)
    hipLaunchKernelGGL((masked_mha_kernel<kDN, kDR, kDV, true>), dim3((unsigned)blocks), dim3(kMThreads), 0,
                       stream, q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, scale * kLog2e, out,
                       lse);
  else
    hipLaunchKernelGGL((masked_mha_kernel<kDN, kDR, kDV, false>), dim3((unsigned)blocks), dim3(kMThreads), 0,
                       stream, q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, scale * kLog2e, out,
                       lse);
}

hipError_t launch_masked_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe, int dn,
                             int dr, int dv, const uint16_t* v, const uint32_t* bits, int words, int T,
                             int S, int H, int64_t q_pos_offset, float scale, uint16_t* out, float* lse,
                             hipStream_t stream) {
  if (T <= 0 || H <= 0) return hipSuccess;
  if (dn == 128 && dr == 64 && dv == 128)
    launch_mha<128, 64, 128>(q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, scale, out, lse, stream);
  else if (dn == 192 && dr == 64 && dv == 256)
    launch_mha<192, 64, 256>(q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, scale, out, lse, stream);
  else
    launch_mha<256, 0, 256>(q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, scale, out, lse, stream);
  return hipGetLastError();
}

}  // namespace dsa
