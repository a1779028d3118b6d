// Exact path of the 128-row attention (grouped routing, and per-token at
// H = 128): recomputes the groups that rows128_attn_kernel marked because a
// score overflowed its fixed softmax reference.  Every other workgroup returns
// at once.
//
// Definition: as rows128_attn_kernel ("[Perf][DSA] Grouped sparse prefill
// with the FlashMLA head-group-mask kernel", commit message and "How"
// section).  This kernel is an online softmax with a running max: when a
// row's max grows by more than 2^8, its O and l are rescaled.  Probabilities
// never exceed 2^8, so no input overflows it.
//
// Design (one workgroup of 8 waves per group, 2 waves per SIMD):
//  * 32-slot tiles of latent rows (D / 8 chunks of 16 B each, LDS rows padded
//    by one chunk) stream through a 3-stage LDS ring by asynchronous global->LDS
//    DMA, issued two tiles ahead; slot indices and membership bytes are
//    wave-uniform and come through scalar loads;
//  * QK^T is split by rows: wave w owns rows 16 w .. 16 w + 15, keeps their
//    queries in registers and computes S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16; masking and the online softmax stay in
//    registers; the bf16 probabilities and per-row rescale factors go to LDS;
//  * PV is split by value columns: wave w owns columns 64 w .. 64 w + 63 of all
//    128 rows and computes O^T = V^T P^T with v_mfma_f32_32x32x16_bf16, V^T
//    from ds_read_b64_tr_b16, P^T from 16-byte reads;
//  * rows with scales (an FP8 latent decoded exactly to bf16): each raw score
//    and each probability is multiplied by its row's scale (scalar loads).
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kGDv = 512;
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGKeys = 32;                            // slots per tile
constexpr int kGStages = 3;
constexpr int kGPStride = 40;                         // halves per probability row (32 + 8 pad)
constexpr float kGSlack = 8.f;                        // lazy-rescale threshold (log2 units)

// D: the latent width, 576 (512 + 64 rope dims) or 512 (no rope part); kScaled: rows carry
// scales (kscale[scale_per_row ? x : 0] for row x)
template <int D, bool kPerToken, bool kScaled>
__global__ __launch_bounds__(kGThreads) void rows128_exact_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ keys, int64_t keys_ld, const int32_t* __restrict__ union_len,
    const uint8_t* __restrict__ hgmask, int T, int H, int S, int ncols, int64_t q_pos_offset,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ ginfo, const float* __restrict__ kscale, int scale_per_row,
    const int32_t* __restrict__ skip) {
  static_assert(D == 576 || D == 512, "latent widths");
  constexpr int kGRowBytes = D * 2 + 16;                          // D / 8 data chunks + 1 pad chunk
  constexpr int kGSlots = kGRowBytes / 16;                        // 73 / 65
  constexpr int kGDma = (kGKeys * kGSlots + 63) / 64;             // wave copies per tile (37 / 33)
  constexpr int kGDmaPerWave = (kGDma + kGWaves - 1) / kGWaves;   // 5 (the rest go to a dummy area)
  constexpr int kGStageBytes = kGDma * 1024;
  static_assert(kGDmaPerWave == 5, "a wave's copies span at most 6 slot rows");
  __shared__ __align__(16) uint8_t stage[kGStages][kGStageBytes];
  __shared__ __align__(16) uint16_t pbuf[128 * kGPStride];
  __shared__ float alpha_s[128];
  __shared__ float linv_s[128];
  __shared__ __align__(16) uint8_t dummy[1024];

  const int G = 128 / H;
  const int NG = (int)gridDim.x;
  const int grp = NG - 1 - xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, n = lane & 15;
  const int2 span = group_span(ginfo, grp, G, T);
  const int t0 = uniform(span.x), ntok = uniform(span.y);
  // only groups the fast kernel marked are recomputed (the mark sits in the LSE of the
  // group's first row)
  if (ntok <= 0 || (skip != nullptr && uniform(*skip) != 0) ||
      __float_as_uint(lse[(size_t)t0 * H]) != kOverflowMark)
    return;

  // the row this lane's wave owns for QK^T / softmax
  const int r_own = 16 * wave + n;
  const int i_own = r_own / H;
  const int h_own = r_own - i_own * H;
  const int tok_own = t0 + i_own;
  const bool row_live = i_own < ntok;

  bf16x8 qreg[D / 32];
  if (row_live) {
    const uint16_t* qrow = q + ((size_t)tok_own * H + h_own) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qreg[s] = bf16x8{};
  }
#pragma unroll
  for (int s = 0; s < D / 32; ++s) asm volatile("" : : "v"(qreg[s]));  // loads done before any copy

  int nkeys;
  if (kPerToken) {
    nkeys = ncols;
  } else {
    nkeys = union_len[grp];
    nkeys = nkeys < 0 ? 0 : (nkeys > ncols ? ncols : nkeys);
  }
  nkeys = uniform(nkeys);
  const int32_t* klist = keys + (size_t)grp * keys_ld;
  const uint8_t* mlist = kPerToken ? nullptr : hgmask + (size_t)grp * keys_ld;
  int64_t pos64 = q_pos_offset + t0;  // per-token mode: the token's position
  if (pos64 > S - 1) pos64 = S - 1;
  const int pos = uniform((int)pos64);
  // validity of slot j0 + r as a latent-row index (grouped: a union entry inside [0, S);
  // per-token: the selection rule) -- wave-uniform, scalar loads
  auto slot_ok = [&](int32_t x, int j) -> bool {
    return j < nkeys && x >= 0 && (kPerToken ? x <= pos : x < S);  // pos <= S - 1
  };
  // the row invalid slots copy (their P is 0): the list's first valid entry (an unselected
  // row may hold anything, and 0 times a NaN is NaN); none: nothing to attend over
  int dummy_row = -1;
  for (int c0 = 0; c0 < nkeys; c0 += 64) {
    const int32_t xv = c0 + lane < nkeys ? klist[c0 + lane] : -1;
    const uint64_t b = ballot(slot_ok(xv, c0 + lane));
    if (b != 0) {
      dummy_row = __builtin_amdgcn_readlane(xv, __builtin_ctzll(b));
      break;
    }
  }
  dummy_row = uniform(dummy_row);
  const int ntiles = dummy_row < 0 ? 0 : (nkeys + kGKeys - 1) / kGKeys;

  // this wave's copies of a tile are 5 w .. 5 w + 4: slots 320 w .. 320 w + 319, i.e. at
  // most 6 consecutive slot rows starting at r_lo
  const int r_lo = uniform((64 * kGDmaPerWave * wave) / kGSlots);
  auto issue = [&](int t) {
    const int j0 = t * kGKeys;
    int32_t x[6];
    const_i32* ip = uniform_const(klist + j0 + r_lo);
    const int avail = min(kGKeys - r_lo, nkeys - j0 - r_lo);  // rows of this tile past r_lo
    if (avail >= 6) {
#pragma unroll
      for (int e = 0; e < 6; ++e) x[e] = ip[e];
    } else {
#pragma unroll
      for (int e = 0; e < 6; ++e) x[e] = e < avail ? ip[e] : -1;
    }
#pragma unroll
    for (int e = 0; e < 6; ++e) x[e] = slot_ok(x[e], j0 + r_lo + e) ? x[e] : dummy_row;
    uint8_t* st = stage[t % kGStages];
#pragma unroll
    for (int u = 0; u < kGDmaPerWave; ++u) {
      const int i = kGDmaPerWave * wave + u;
      if (i < kGDma) {
        const int r0 = (64 * i) / kGSlots;
        const int thr = kGSlots * (r0 + 1) - 64 * i;
        const bool up = lane >= thr;
        const int r = up ? r0 + 1 : r0;
        const int c = 64 * i + lane - kGSlots * r;
        const int e0 = r0 - r_lo;  // 0..4, wave-uniform
        int32_t x0 = x[0], x1 = x[1];
#pragma unroll
        for (int e = 1; e < 5; ++e) {
          x0 = e == e0 ? x[e] : x0;
          x1 = e == e0 ? x[e + 1] : x1;
        }
        int32_t xr = up ? x1 : x0;
        if (r >= kGKeys) xr = 0;
        dma16(kv + (size_t)xr * D + (c < D / 8 ? c : 0) * 8, lds_addr(st + 1024 * i));
      } else {
        dma16(kv, lds_addr(dummy));  // keeps every wave's copy count per tile equal
      }
    }
  };

  // for the row this lane owns: bit 4 kb + jj <-> slot 16 kb + 4 g + jj of tile t is allowed;
  // kScaled: ksc[kb][jj] = that slot's row scale
  auto allowed_bits = [&](int t, f32x4 (&ksc)[2]) -> uint32_t {
    const int j0 = t * kGKeys;
    uint32_t bits = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int jb = j0 + 16 * kb;
      const_i32* ip = uniform_const(klist + jb);
      int32_t e[16];
      if (!kPerToken || nkeys - jb >= 16) {  // union lists are padded to whole tiles
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = ip[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = r < nkeys - jb ? ip[r] : -1;
      }
      uint32_t vbits = 0;  // validity of the 16 slots
#pragma unroll
      for (int r = 0; r < 16; ++r) vbits |= slot_ok(e[r], jb + r) ? (1u << r) : 0u;
      if (kScaled) {  // (uniform indices: scalar loads)
        const_i32* sp = uniform_const(reinterpret_cast<const int32_t*>(kscale));
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = __int_as_float(sp[scale_per_row && ((vbits >> r) & 1u) ? e[r] : 0]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ksc[kb][jj] = g == 0 ? v[jj] : g == 1 ? v[4 + jj] : g == 2 ? v[8 + jj] : v[12 + jj];
      }
      const uint32_t vb = (vbits >> (4 * g)) & 0xfu;
      if (kPerToken) {
        bits |= vb << (4 * kb);
      } else {
        // membership bytes of slots 16 kb + 4 g .. + 3
        const_i32* mp = uniform_const(reinterpret_cast<const int32_t*>(mlist + jb));
        const uint32_t w0 = (uint32_t)mp[0], w1 = (uint32_t)mp[1], w2 = (uint32_t)mp[2], w3 = (uint32_t)mp[3];
        const uint32_t w = g == 0 ? w0 : g == 1 ? w1 : g == 2 ? w2 : w3;
        uint32_t mbits = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) mbits |= ((w >> (8 * jj + i_own)) & 1u) << jj;
        bits |= (vb & mbits) << (4 * kb);
      }
    }
    return bits;
  };

  float m_run = kNegInf, l_run = 0.f;  // row r_own (replicated over the 4 lane groups)
  f32x16 o[2][4];                      // [col block][row block]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) o[cb][rb] = f32x16{};

  const int hi = lane >> 5, m = lane & 31;
  const int koff = n * kGRowBytes + 16 * g;  // K read: row n of a 16-slot block, chunk 4 s + g
  // transposed V reads: row 8 hi + s16 / 4 (+4), columns 64 w + 32 cb + 16 (g16 % 2) + 4 (s16 % 4)
  const int voff = (8 * hi + ((lane & 15) >> 2)) * kGRowBytes +
                   2 * (64 * wave + 16 * (g & 1) + 4 * (lane & 3));
  const int poff = m * kGPStride + 8 * hi;   // P^T read: row 32 rb + m, slots 16 ks + 8 hi .. + 8

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles)
      wait_vmcnt<kGDmaPerWave>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // tile t visible; every wave is done with tile t - 1 (stage and P)
    if (t + 2 < ntiles) issue(t + 2);
    f32x4 ksc[2] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
    const uint32_t abits = allowed_bits(t, ksc);

    const uint8_t* tile = stage[t % kGStages];
    // ---- scores of this wave's 16 rows over the 32 slots
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = mfma16x16x32(*reinterpret_cast<const bf16x8*>(tile + koff + kb * 16 * kGRowBytes + 64 * s),
                                qreg[s], sacc[kb]);
    // sacc[kb][jj] = score(slot 16 kb + 4 g + jj, row r_own)

    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bool ok = ((abits >> (4 * kb + jj)) & 1u) != 0u;
        const float raw = kScaled ? sacc[kb][jj] * ksc[kb][jj] : sacc[kb][jj];
        const float val = ok ? raw * scale_log2 : kNegInf;
        sacc[kb][jj] = val;
        mt = fmaxf(mt, val);
      }
    }
    mt = max_over_rowgroups(mt);
    float alpha = 1.f;
    const bool need = mt > m_run + kGSlack;
    if (ballot(need) != 0) {
      const float m_new = need ? mt : m_run;
      alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
      m_run = m_new;
    }
    const float msafe = m_run == kNegInf ? 0.f : m_run;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x4 pw;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p = fast_exp2(sacc[kb][jj] - msafe);
        ls += p;
        pw[jj] = (__bf16)(kScaled ? p * ksc[kb][jj] : p);
      }
      *reinterpret_cast<bf16x4*>(pbuf + r_own * kGPStride + 16 * kb + 4 * g) = pw;
    }
    l_run += sum_over_rowgroups(ls);
    if (g == 0) alpha_s[r_own] = alpha;
    __syncthreads();  // P and alpha of all 128 rows visible

    // ---- O^T[64 w .. 64 w + 63][all rows] += V^T P^T over the 32 slots
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const float al = alpha_s[32 * rb + m];
      if (ballot(al != 1.f) != 0) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) o[cb][rb] *= al;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 va[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint8_t* vp = tile + voff + 16 * ks * kGRowBytes + 64 * cb;
        const u16x4 lo = lds_read_tr16(vp);
        const u16x4 up = lds_read_tr16(vp + 4 * kGRowBytes);
        va[cb] = __builtin_bit_cast(bf16x8, u16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8 pb = *reinterpret_cast<const bf16x8*>(pbuf + 32 * rb * kGPStride + poff + 16 * ks);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) o[cb][rb] = mfma32x32x16(va[cb], pb, o[cb][rb]);
      }
    }
  }

  if (g == 0) {
    linv_s[r_own] = l_run > 0.f ? 1.f / l_run : 0.f;
    if (row_live)
      lse[(size_t)tok_own * H + h_own] = l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
  }
  __syncthreads();

  // o[cb][rb][j] = O^T[col 64 w + 32 cb + 8 (j / 4) + 4 hi + j % 4][row 32 rb + m]
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = 32 * rb + m;
    const int i = row / H;
    const int h = row - i * H;
    const int tok = t0 + i;
    if (i >= ntok) continue;
    const float inv = linv_s[row];
    uint16_t* orow = out + ((size_t)tok * H + h) * kGDv + 64 * wave + 4 * hi;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bf16x4 w = {(__bf16)(o[cb][rb][4 * jj + 0] * inv), (__bf16)(o[cb][rb][4 * jj + 1] * inv),
                          (__bf16)(o[cb][rb][4 * jj + 2] * inv), (__bf16)(o[cb][rb][4 * jj + 3] * inv)};
        *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * jj) = w;
      }
  }
}

template <int D, bool kPerToken, bool kScaled>
static void launch_exact(int blocks, hipStream_t stream, const uint16_t* q, const uint16_t* kv, const int32_t* keys,
                         int64_t keys_ld, const int32_t* union_len, const uint8_t* hgmask, int T, int H, int S,
                         int ncols, int64_t q_pos_offset, float sl, uint16_t* out, float* lse,
                         const int32_t* ginfo, const float* kscale, int scale_per_row, const int32_t* skip) {
  hipLaunchKernelGGL((rows128_exact_kernel<D, kPerToken, kScaled>), dim3(blocks), dim3(kGThreads), 0, stream, q, kv,
                     keys, keys_ld, union_len, hgmask, T, H, S, ncols, q_pos_offset, sl, out, lse, ginfo, kscale,
                     scale_per_row, skip);
}

template <int D, bool kPerToken>
static void launch_exact_scaled(int blocks, hipStream_t stream, const uint16_t* q, const uint16_t* kv,
                                const int32_t* keys, int64_t keys_ld, const int32_t* union_len,
                                const uint8_t* hgmask, int T, int H, int S, int ncols, int64_t q_pos_offset,
                                float sl, uint16_t* out, float* lse, const int32_t* ginfo, const float* kscale,
                                int scale_per_row, const int32_t* skip) {
  if (kscale)
    launch_exact<D, kPerToken, true>(blocks, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                     q_pos_offset, sl, out, lse, ginfo, kscale, scale_per_row, skip);
  else
    launch_exact<D, kPerToken, false>(blocks, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                      q_pos_offset, sl, out, lse, ginfo, kscale, scale_per_row, skip);
}

hipError_t launch_rows128_exact(const uint16_t* q, const uint16_t* kv, const int32_t* keys,
                                int64_t keys_ld, const int32_t* union_len, const uint8_t* hgmask,
                                int T, int H, int S, int ncols, int64_t q_pos_offset, float scale,
                                uint16_t* out, float* lse, hipStream_t stream, const int32_t* group_info,
                                int ngroups, int d_qk, const float* kscale, int scale_per_row,
                                const int32_t* skip) {
  const int NG = ngroups;
  if (NG == 0) return hipSuccess;
  const float sl = scale * kLog2e;
  if (d_qk == 512) {
    if (hgmask != nullptr)
      launch_exact_scaled<512, false>(NG, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                      q_pos_offset, sl, out, lse, group_info, kscale, scale_per_row, skip);
    else
      launch_exact_scaled<512, true>(NG, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                     q_pos_offset, sl, out, lse, group_info, kscale, scale_per_row, skip);
  } else {
    if (hgmask != nullptr)
      launch_exact_scaled<576, false>(NG, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                      q_pos_offset, sl, out, lse, group_info, kscale, scale_per_row, skip);
    else
      launch_exact_scaled<576, true>(NG, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                     q_pos_offset, sl, out, lse, group_info, kscale, scale_per_row, skip);
  }
  return hipGetLastError();
}

}  // namespace dsa
