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
// MI355X design (one workgroup of 4 waves per (256-query tile, head); one wave
// per SIMD with the full register file):
//  * each wave owns 64 query rows as two 32-row blocks; their queries sit in
//    registers as the B operands of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, the
//    full-rate shape on gfx950) and O^T (2 x 32 x kDV) sits in accumulation
//    registers; each V^T operand read from LDS feeds both blocks;
//  * 32-key tiles of K and V (one head's rows) and the matching mask words
//    stream through a 4-stage LDS ring by asynchronous global->LDS DMA, two
//    tiles ahead of the compute; one barrier per tile.  Each wave copy moves
//    128 B of 8 consecutive key rows into the swizzled 8-row-group layout
//    (common.h), addressed as a uniform base plus the lane's 32-bit offset, so
//    every operand read is a per-lane base plus an immediate with no LDS bank
//    conflicts;
//  * the PV runs one tile behind the QK, and the softmax work sits between the
//    MFMAs of the same wave, so the vector ALU works while the matrix cores
//    do: the QK MFMAs of tile t take block 1's exponentials of tile
//    t-1 (block 1's new scores go to a second buffer, so each K operand read
//    feeds both blocks); tile t-1's PV MFMAs take tile t's masking and maxima
//    and block 0's exponentials;
//  * the causal test and the top-k bit select scores in registers (bit-field
//    insert of -inf); the softmax scale is folded into one fused multiply-add
//    before the base-2 exponential; the bf16 probabilities go straight from
//    the accumulators into the B operand of O^T = V^T P^T (keys relabelled
//    consistently), V^T comes from ds_read_b64_tr_b16;
//  * fixed-reference softmax: a row's reference is the max of its first tile
//    with a selected key and never moves, so O^T is never rescaled (a VALU
//    rescale would pull the accumulators out of the accumulation registers);
//    exponents stay below 2^64 unless a later score exceeds the reference by
//    more than that, in which case the row is marked (LSE = +inf) and the
//    exact path below recomputes its 256-query tile with a running max;
//  * key tiles past the causal diagonal of the tile's last query are never
//    visited; query tiles run longest first.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kMWaves = 4;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMQ = 64 * kMWaves;                     // query rows per workgroup (64 per wave)
constexpr int kMKeys = 32;                            // keys per tile
constexpr int kMStages = 4;
constexpr float kMRefSlack = 64.f;                    // reference range: exponents up to 2^64

// (The QK MFMAs are written out -- mfma_qk_first / mfma_qk, common.h -- so that their S^T
// accumulators stay in VGPRs while O^T takes the accumulation registers.  Every VALU access
// to their results comes at least one 16-MFMA chain later.)

// Geometry (kDN, kDR, kDV): the key is k_nope (kDN dims, per head) followed by k_pe (kDR
// dims, shared by every head), the value kDV dims per head: (256, 0, 256) NoPE -- K is
// k_nope itself; (192, 64, 256); (128, 64, 128).
// kDense: plain causal attention (every causal key selected): no mask words are copied.
template <int kDN, int kDR, int kDV, bool kDense>
__global__ __launch_bounds__(kMThreads) void masked_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kpe,
    const uint16_t* __restrict__ v, const uint32_t* __restrict__ bits, int words, int T, int S,
    int H, int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int kDQK = kDN + kDR;
  static_assert(kDN % 64 == 0 && kDR % 64 == 0 && kDV % 64 == 0, "whole 128-byte blocks per row");
  constexpr int kKBlocks = kDQK / 64, kVBlocks = kDV / 64;  // 1 KiB blocks per 8-row group
  constexpr int kNBlocks = kDN / 64;                        // ... of them from k_nope
  constexpr int kKGroupBytes = 1024 * kKBlocks, kVGroupBytes = 1024 * kVBlocks;
  constexpr int kKTileBytes = 4 * kKGroupBytes;         // 32 keys of K
  constexpr int kStageBytes = kKTileBytes + 4 * kVGroupBytes;
  constexpr int kQSteps = kDQK / 16;                    // k-steps of S^T = K Q^T
  constexpr int kCB = kDV / 32;                         // O^T column blocks
  constexpr int kPVSteps = 2 * kCB;                     // V^T operands per tile
  // copies per wave per tile: its 8-row group of K and of V, + the mask-word copy
  constexpr int kOps = kKBlocks + kVBlocks + (kDense ? 0 : 1);
  __shared__ __align__(16) uint8_t stage[kMStages][kStageBytes];
  __shared__ __align__(16) uint32_t maskw[kDense ? 1 : kMStages][kMWaves][64];

  // longest query tiles first; consecutive blocks take consecutive heads, so the
  // round-robin XCD dispatch keeps each head on one XCD and balances the work
  const int nqt = (T + kMQ - 1) / kMQ;
  const int lb = (int)blockIdx.x;
  const int qt = nqt - 1 - lb / H;
  const int h = lb - (lb / H) * H;
  const int q0 = qt * kMQ;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;  // (wave: a scalar)
  const int hi = lane >> 5, m = lane & 31;
  // this lane's rows: block 0 = ra, block 1 = ra + 32
  const int ra = q0 + 64 * wave + m, rb = ra + 32;
  // last key a row may see (positions beyond S - 1 cannot be selected); -1 for rows >= T
  auto last_key = [&](int row) -> int {
    int64_t p = q_pos_offset + row;
    if (p > S - 1) p = S - 1;
    return row < T ? (int)p : -1;
  };
  const int rposa = last_key(ra), rposb = last_key(rb);

  // queries; a negative scale is applied as |scale| on negated queries so that the
  // running max can be taken on raw scores
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sc = fabsf(scale_log2);
  bf16x8 qa[kQSteps], qb[kQSteps];
  {
    // (rows past T load row T - 1 and are zeroed after: unconditional loads go out back to
    // back, where a load under a branch is waited for inside it)
    const uint16_t* qra = q + ((size_t)min(ra, T - 1) * H + h) * kDQK + 8 * hi;
    const uint16_t* qrb = q + ((size_t)min(rb, T - 1) * H + h) * kDQK + 8 * hi;
    uint4 la[kQSteps], lb[kQSteps];
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      la[s] = *reinterpret_cast<const uint4*>(qra + 16 * s);
      lb[s] = *reinterpret_cast<const uint4*>(qrb + 16 * s);
    }
    const uint32_t ka = ra < T ? 0xffffffffu : 0u, kb = rb < T ? 0xffffffffu : 0u;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      uint4 wa = la[s], wb = lb[s];
      wa.x = (wa.x ^ qsign) & ka; wa.y = (wa.y ^ qsign) & ka; wa.z = (wa.z ^ qsign) & ka; wa.w = (wa.w ^ qsign) & ka;
      wb.x = (wb.x ^ qsign) & kb; wb.y = (wb.y ^ qsign) & kb; wb.z = (wb.z ^ qsign) & kb; wb.w = (wb.w ^ qsign) & kb;
      qa[s] = __builtin_bit_cast(bf16x8, wa);
      qb[s] = __builtin_bit_cast(bf16x8, wb);
    }
  }
  // complete the query loads now, before any asynchronous copy is in flight
#pragma unroll
  for (int s = 0; s < kQSteps; ++s) asm volatile("" : : "v"(qa[s]), "v"(qb[s]));

  const int last = min(T, q0 + kMQ) - 1;
  int64_t kend64 = q_pos_offset + last + 1;
  if (kend64 > S) kend64 = S;
  const int kend = (int)kend64;
  const int ntiles = (kend + kMKeys - 1) / kMKeys;

  // copies: wave w fills rows 8 w .. 8 w + 7 of the K tile and of the V tile; lane l takes
  // row l / 8 of the group, position l % 8 (chunk 8 c + pos ^ swizzle).  Each row is a
  // uniform tile base plus the lane's 32-bit offset (a tile spans < 2^31 bytes).
  const int crow = 8 * wave + (lane >> 3);
  const int cchunk = (lane & 7) ^ swz8(lane >> 3) ^ wave;
  const uint32_t kstride = (uint32_t)H * kDN * 2, vstride = (uint32_t)H * kDV * 2;
  const uint32_t pstride = kDR * 2;
  const uint8_t* kb0 = reinterpret_cast<const uint8_t*>(k + (size_t)h * kDN);
  const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(v + (size_t)h * kDV);
  const uint8_t* pb0 = reinterpret_cast<const uint8_t*>(kpe);
  // mask words: lane l copies row q0 + 64 w + l (block l / 32, row l % 32)
  const int mrow = min(q0 + 64 * wave + lane, T - 1);
  const uint32_t* mrowp = kDense ? bits : bits + (size_t)mrow * words;

  auto issue = [&](int t) {
    const int rr = min(crow, kend - 1 - kMKeys * t);  // (keys past kend repeat the last one)
    const size_t key0 = (size_t)kMKeys * t;
    const uint32_t dst = lds_addr(stage[t % kMStages]) + wave * kKGroupBytes;
    const uint32_t vdst = lds_addr(stage[t % kMStages]) + kKTileBytes + wave * kVGroupBytes;
    const uint32_t ko = (uint32_t)rr * kstride + 16 * cchunk;
    const uint8_t* kbt = kb0 + key0 * kstride;
#pragma unroll
    for (int c = 0; c < kNBlocks; ++c) dma16_sbase(ko, kbt + 128 * c, dst + 1024 * c);
    if constexpr (kDR > 0) {
      const uint32_t po = (uint32_t)rr * pstride + 16 * cchunk;
      const uint8_t* pbt = pb0 + key0 * pstride;
#pragma unroll
      for (int c = kNBlocks; c < kKBlocks; ++c) dma16_sbase(po, pbt + 128 * (c - kNBlocks), dst + 1024 * c);
    }
    const uint32_t vo = (uint32_t)rr * vstride + 16 * cchunk;
    const uint8_t* vbt = vb0 + key0 * vstride;
#pragma unroll
    for (int c = 0; c < kVBlocks; ++c) dma16_sbase(vo, vbt + 128 * c, vdst + 1024 * c);
    if constexpr (!kDense) dma4(mrowp + t, lds_addr(&maskw[t % kMStages][wave][0]));
  };

  // online softmax state per block (m: reference max of the exponents, log2 units)
  float ma = kNegInf, mb = kNegInf, la = 0.f, lb_ = 0.f, nma = 0.f, nmb = 0.f;
  bool fba = false, fbb = false;  // a later max left the reference's range: exact path
  f32x16 oa[kCB], ob[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    oa[cb] = f32x16{};
    ob[cb] = f32x16{};
  }
  f32x16 sa, sb;               // S^T of the current tile (masked in place)
  bf16x8 pa[2], pan[2], pb[2];  // bf16 P^T operands (pan: block 0's next tile)

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

  using yes = std::true_type;
  using no = std::false_type;

  // ---- softmax pieces (VALU), placed between MFMAs below ----
  // scores: sacc[j] = raw score(key k0 + 8 (j / 4) + 4 hi + j % 4, row)
  uint32_t alla = 0u, allb = 0u;
  float lsa = 0.f, lsb = 0.f;
  // allowed keys of tile t: top-k bit AND key <= position; bit kk <-> key k0 + 4 hi + kk
  auto mask_setup = [&](int t) {
    const int k0 = t * kMKeys;
    const int lima = rposa - k0 - 4 * hi, limb = rposb - k0 - 4 * hi;
    alla = lima >= 31 ? 0xffffffffu : (lima < 0 ? 0u : ((2u << lima) - 1u));
    allb = limb >= 31 ? 0xffffffffu : (limb < 0 ? 0u : ((2u << limb) - 1u));
    if constexpr (!kDense) {
      const uint8_t* mw = reinterpret_cast<const uint8_t*>(&maskw[0][wave][m]) +
                          loop_local((t % kMStages) * (int)sizeof(maskw[0]));
      alla &= *reinterpret_cast<const uint32_t*>(mw) >> (4 * hi);
      allb &= *reinterpret_cast<const uint32_t*>(mw + 128) >> (4 * hi);
    }
  };
  auto select = [&](f32x16& c, uint32_t allowed, int j) {
    const int kk = 8 * (j >> 2) + (j & 3);
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)allowed, kk, 1);  // all ones if allowed
    // (the element goes through a scalar first: a bit cast applied directly to a
    // vector element reads element 0 with this compiler)
    const float raw = c[j];
    const float val =
        __builtin_bit_cast(float, (sel & __builtin_bit_cast(uint32_t, raw)) | (~sel & 0xff800000u));
    c[j] = val;
  };
  // fixed reference: a row's reference is the max of its first tile with a selected key
  // (O^T and l are still zero then) and never moves, so O^T is never rescaled; a later max
  // beyond reference + 2^kMRefSlack marks the row for the exact path.  Maxima are taken only
  // while a row of the wave has no reference (need_ref, normally the first tiles); after that
  // a score that far above the reference shows in the row's sum, which is checked at the end.
  bool need_ref = true;
  auto reduce = [&](const f32x16& c, float& mref, float& nm, bool& fb) {
    if (!need_ref) return;  // (a uniform branch around the whole reduction)
    float mt = c[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mt = fmaxf(mt, c[j]);
    mt = max_xor32(mt) * sc;
    fb = fb | ((mref != kNegInf) & (mt > mref + kMRefSlack));  // (no short circuit: no branch)
    mref = mref == kNegInf ? mt : mref;
    nm = mref == kNegInf ? 0.f : -mref;
  };
  auto expo = [&](const f32x16& c, float nm, float& ls, bf16x8* p, int j) {
    const float e = fast_exp2(__builtin_fmaf(c[j], sc, nm));
    ls += e;
    p[j >> 3][j & 7] = (__bf16)e;
  };
  // mask/max work of a tile, then block 0's exponentials, as 50 numbered pieces
  constexpr int kTasks = 16 + 1 + 16 + 1 + 16;
  auto task = [&](int id) {
    if (id < 16)
      select(sa, alla, id);
    else if (id == 16)
      reduce(sa, ma, nma, fba);
    else if (id < 33)
      select(sb, allb, id - 17);
    else if (id == 33)
      reduce(sb, mb, nmb, fbb);
    else
      expo(sa, nma, lsa, pan, id - 34);
  };

  // Phase 1 of tile t: S^T of both blocks (kS; one K operand read feeds both MFMAs of a
  // k-step), block 1's into a second buffer, interleaved with block 1's exponentials of the
  // previous tile (kE; its masked scores are in sb); then sb takes the new scores.
  f32x16 sbn;
  auto phase1 = [&](auto do_s, auto do_exp, int t) {
    constexpr bool kS = decltype(do_s)::value, kE = decltype(do_exp)::value;
    const uint8_t* kt = &stage[0][0] + loop_local((t % kMStages) * kStageBytes);
    auto kread = [&](int s) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(kt + kofs[s & 3] + 1024 * (s >> 2));
    };
    constexpr int kAhead = 2;
    bf16x8 kw[kAhead];
    if constexpr (kS) {
#pragma unroll
      for (int s = 0; s < kAhead; ++s) kw[s] = kread(s);
    }
    lsb = 0.f;
    constexpr int kSteps = kS ? kQSteps : 16;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kS) sa = s == 0 ? mfma_qk_first(kw[s % kAhead], qa[s]) : mfma_qk(kw[s % kAhead], qa[s], sa);
      if constexpr (kE) {
#pragma unroll
        for (int j = s * 16 / kSteps; j < (s + 1) * 16 / kSteps; ++j) expo(sb, nmb, lsb, pb, j);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kS) {
        sbn = s == 0 ? mfma_qk_first(kw[s % kAhead], qb[s]) : mfma_qk(kw[s % kAhead], qb[s], sbn);
        if (s + kAhead < kQSteps) kw[s % kAhead] = kread(s + kAhead);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kE) lb_ += lsb;  // this half's keys; the halves are summed at the end
    if constexpr (kS) sb = sbn;
  };

  // Phase 2: O^T += V^T P^T for tile tv (kP; one V^T operand read per MFMA pair)
  // interleaved with the softmax pieces of tile t (kM).
  auto phase2 = [&](auto do_pv, auto do_mask, int tv, int t) {
    constexpr bool kP = decltype(do_pv)::value, kM = decltype(do_mask)::value;
    const uint8_t* vt = &stage[0][0] + loop_local((tv % kMStages) * kStageBytes) + kKTileBytes;
    // step st covers keys 16 st .. 16 st + 15 with k-slot (hi, i) <-> key 16 st + 8 (i / 4) +
    // 4 hi + i % 4, i.e. accumulator registers 8 st .. 8 st + 7; MFMA pair i is step i / kCB,
    // column block i % kCB
    auto vread = [&](int i) -> bf16x8 {
      const int st = i / kCB, cbk = i % kCB;
      // rows 16 st + 8 uu + vr8 are in group 2 st + uu; chunk 4 cb + c2 is in block cb / 2
      const int p0 = 16 * (vx ^ (4 * (cbk & 1)) ^ (2 * st));
      const int p1 = 16 * (vx ^ (4 * (cbk & 1)) ^ (2 * st + 1));
      const u16x4 lo = lds_read_tr16(vt + (2 * st) * kVGroupBytes + 1024 * (cbk >> 1) + vbase + p0);
      const u16x4 up = lds_read_tr16(vt + (2 * st + 1) * kVGroupBytes + 1024 * (cbk >> 1) + vbase + p1);
      return __builtin_bit_cast(bf16x8, u16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    constexpr int kVAhead = 2;
    bf16x8 vw[kVAhead];
    if constexpr (kP) {
#pragma unroll
      for (int i = 0; i < kVAhead; ++i) vw[i] = vread(i);
    }
    if constexpr (kM) {
      mask_setup(t);
      lsa = 0.f;
    }
    constexpr int kSlots = kP ? 2 * kPVSteps : kTasks;
#pragma unroll
    for (int c = 0; c < kSlots; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kP) {
        const int i = c >> 1;
        if ((c & 1) == 0) {
          oa[i % kCB] = mfma32x32x16(vw[i % kVAhead], pa[i / kCB], oa[i % kCB]);
        } else {
          ob[i % kCB] = mfma32x32x16(vw[i % kVAhead], pb[i / kCB], ob[i % kCB]);
          if (i + kVAhead < kPVSteps) vw[i % kVAhead] = vread(i + kVAhead);
        }
      }
      if constexpr (kM) {
#pragma unroll
        for (int id = c * kTasks / kSlots; id < (c + 1) * kTasks / kSlots; ++id) task(id);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kM) {
      la += lsa;
      pa[0] = pan[0];
      pa[1] = pan[1];
    }
  };

  // Tile t: wait for its copies (the next tile's stay in flight), barrier, copy tile t + 2
  // into the stage that tile t - 2 used (its V was read in the previous tile's step).
  auto arrive = [&](int t) {
    if (t + 1 >= ntiles)
      wait_vmcnt<0>();
    else
      wait_vmcnt<kOps>();
    __syncthreads();
    if (t + 2 < ntiles) issue(t + 2);
  };

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 0) {
    arrive(0);
    phase1(yes{}, no{}, 0);
    phase2(no{}, yes{}, 0, 0);
  }
  // steady state: tile t's QK, tile t - 1's PV, tile t's softmax around them
  for (int t = 1; t < ntiles; ++t) {
    need_ref = need_ref && ballot(ma == kNegInf || mb == kNegInf) != 0;
    arrive(t);
    phase1(yes{}, yes{}, t);
    phase2(yes{}, yes{}, t - 1, t);
  }
  // last tile: block 1's exponentials, then its PV
  if (ntiles > 0) {
    phase1(no{}, yes{}, ntiles - 1);
    phase2(yes{}, no{}, ntiles - 1, ntiles - 1);
  }

  // o[cb][j] = O^T[col 32 cb + 8 (j / 4) + 4 hi + j % 4][row]
  // (rows marked for the exact path get LSE = +inf, which no finite softmax produces)
  auto store = [&](int row, float l, float mref, bool fb, const f32x16* o) {
    const float l_tot = sum_xor32(l);  // (every lane takes part)
    // every probability is at most 2^kMRefSlack unless a score rose that far above the
    // row's reference: then its sum shows it (an infinite or NaN sum as well)
    fb = fb || !(l_tot <= __builtin_ldexpf(1.f, (int)kMRefSlack));
    if (row >= T) return;
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
      lse[(size_t)row * H + h] = fb ? __builtin_inff() : l_tot > 0.f ? (mref + fast_log2(l_tot)) * kLn2 : kNegInf;
  };
  store(ra, la, ma, fba, oa);
  store(rb, lb_, mb, fbb, ob);
}

// ---------------------------------------------------------------------------
// Exact path: running-max softmax (the reference moves whenever a tile's max exceeds it
// by more than 2^8, rescaling O^T and l), 8 waves x 32 query rows per (256-query tile,
// head), 2 waves per SIMD, 3-stage ring with 4 query k-steps in LDS.  Launched after the
// fast kernel with recheck = 1, a workgroup returns at once unless one of its rows is
// marked; launched with recheck = 0 it computes every tile.
// ---------------------------------------------------------------------------
constexpr int kXWaves = 8;
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXQ = 32 * kXWaves;                     // query rows per workgroup
constexpr int kXKeys = 32;
constexpr int kXStages = 3;
constexpr float kXRescaleSlack = 8.f;                 // rescale O only when the max grows by > 2^8
constexpr int kXQRegMax = 12;                         // query k-steps kept in registers (at most)
static_assert(kXQ == kMQ, "both paths tile the queries alike");

template <int kDN, int kDR, int kDV, bool kDense>
__global__ __launch_bounds__(kXThreads) void masked_mha_exact_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kpe,
    const uint16_t* __restrict__ v, const uint32_t* __restrict__ bits, int words, int T, int S,
    int H, int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int recheck) {
  constexpr int kDQK = kDN + kDR;
  static_assert(kDN % 64 == 0 && kDR % 64 == 0 && kDV % 64 == 0, "whole 128-byte blocks per row");
  constexpr int kKBlocks = kDQK / 64, kVBlocks = kDV / 64;  // 1 KiB blocks per 8-row group
  constexpr int kKGroupBytes = 1024 * kKBlocks, kVGroupBytes = 1024 * kVBlocks;
  constexpr int kKTileBytes = 4 * kKGroupBytes;         // 32 keys of K
  constexpr int kStageBytes = kKTileBytes + 4 * kVGroupBytes;
  constexpr int kQSteps = kDQK / 16;                    // k-steps of S^T = K Q^T
  constexpr int kQRegSteps = kQSteps < kXQRegMax ? kQSteps : kXQRegMax;
  constexpr int kQLdsSteps = kQSteps - kQRegSteps;      // the rest sit in LDS (lane-private)
  constexpr int kCB = kDV / 32;                         // O^T column blocks
  // copies per wave per tile (K waves 0..3, V waves 4..7), + the mask-word copy
  constexpr int kOpsK = kKBlocks + (kDense ? 0 : 1), kOpsV = kVBlocks + (kDense ? 0 : 1);
  __shared__ __align__(16) uint8_t stage[kXStages][kStageBytes];
  __shared__ __align__(16) uint32_t maskw[kDense ? 1 : kXStages][kXWaves][64];
  __shared__ __align__(16) uint4 qlds[kXWaves][kQLdsSteps > 0 ? kQLdsSteps : 1][64];

  // longest query tiles first; consecutive blocks take consecutive heads, so the
  // round-robin XCD dispatch keeps each head on one XCD and balances the work
  const int nqt = (T + kXQ - 1) / kXQ;
  const int lb = (int)blockIdx.x;
  const int qt = nqt - 1 - lb / H;
  const int h = lb - (lb / H) * H;
  const int q0 = qt * kXQ;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;  // (wave: a scalar)
  if (recheck) {
    // only tiles with a row marked by the fast kernel (LSE +inf or NaN) are recomputed
    bool marked = false;
    if (tid < kXQ && q0 + tid < T) marked = !(lse[(size_t)(q0 + tid) * H + h] < __builtin_inff());
    if (__syncthreads_or(marked) == 0) return;
  }
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

  const int last = min(T, q0 + kXQ) - 1;
  int64_t kend64 = q_pos_offset + last + 1;
  if (kend64 > S) kend64 = S;
  const int kend = (int)kend64;
  const int ntiles = (kend + kXKeys - 1) / kXKeys;
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
    int key = t * kXKeys + crow;
    key = key < kend ? key : kend - 1;
    const uint16_t* src = cbase + (size_t)key * key_stride;
    const uint16_t* psrc = kDR > 0 ? pbase + (size_t)key * kDR : src;
    const uint32_t dst = lds_addr(stage[t % kXStages]) + cdst;
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
      dma4(bits + (size_t)mrow * words + ((t * kXKeys) >> 5), lds_addr(&maskw[t % kXStages][wave][0]));
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
    const int sofs = loop_local((t % kXStages) * kStageBytes);
    const uint8_t* kt = &stage[0][0] + sofs;
    const uint8_t* vt = kt + kKTileBytes;
    const int k0 = t * kXKeys;

    // K operand reads run kXAhead steps ahead of the MFMAs (the order is pinned: left to
    // itself the scheduler puts every read right before its MFMA and waits out its latency)
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(&qlds[wave][0][0]) + loop_local(16 * lane);
    auto kread = [&](int s) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(kt + kofs[s & 3] + 1024 * (s >> 2));
    };
    auto qread = [&](int s) -> bf16x8 {
      return s < kQRegSteps ? qreg[s < kQRegSteps ? s : 0]
                            : *reinterpret_cast<const bf16x8*>(qb + 1024 * (s - kQRegSteps));
    };
    constexpr int kXAhead = 4;
    bf16x8 kw[kXAhead], qw[kXAhead];
#pragma unroll
    for (int s = 0; s < kXAhead; ++s) {
      kw[s] = kread(s);
      qw[s] = qread(s);
    }
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      sacc = mfma32x32x16(kw[s % kXAhead], qw[s % kXAhead], sacc);
      if (s + kXAhead < kQSteps) {
        kw[s % kXAhead] = kread(s + kXAhead);
        qw[s % kXAhead] = qread(s + kXAhead);
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
                       loop_local((t % kXStages) * (int)sizeof(maskw[0]))) >> (4 * hi);
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
    const bool need = mt > m_run + kXRescaleSlack;
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
    // kXVAhead MFMAs ahead (order pinned as for QK)
    auto vread = [&](int i) -> bf16x8 {
      const int st = i / kCB, cb = i % kCB;
      // rows 16 st + 8 uu + vr8 are in group 2 st + uu; chunk 4 cb + c2 is in block cb / 2
      const int p0 = 16 * (vx ^ (4 * (cb & 1)) ^ (2 * st));
      const int p1 = 16 * (vx ^ (4 * (cb & 1)) ^ (2 * st + 1));
      const u16x4 lo = lds_read_tr16(vt + (2 * st) * kVGroupBytes + 1024 * (cb >> 1) + vbase + p0);
      const u16x4 up = lds_read_tr16(vt + (2 * st + 1) * kVGroupBytes + 1024 * (cb >> 1) + vbase + p1);
      return __builtin_bit_cast(bf16x8, u16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    constexpr int kXVAhead = 3;
    bf16x8 vw[kXVAhead];
#pragma unroll
    for (int i = 0; i < kXVAhead; ++i) vw[i] = vread(i);
#pragma unroll
    for (int i = 0; i < 2 * kCB; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      o[i % kCB] = mfma32x32x16(vw[i % kXVAhead], bop[i / kCB], o[i % kCB]);
      if (i + kXVAhead < 2 * kCB) vw[i % kXVAhead] = vread(i + kXVAhead);
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
  const float sl = scale * kLog2e;
  // no membership bits: every causal key is selected (plain causal attention); the exact
  // pass then redoes the tiles with marked rows
  if (bits == nullptr) {
    hipLaunchKernelGGL((masked_mha_kernel<kDN, kDR, kDV, true>), dim3((unsigned)blocks), dim3(kMThreads), 0,
                       stream, q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, sl, out, lse);
    hipLaunchKernelGGL((masked_mha_exact_kernel<kDN, kDR, kDV, true>), dim3((unsigned)blocks), dim3(kXThreads),
                       0, stream, q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, sl, out, lse, 1);
  } else {
    hipLaunchKernelGGL((masked_mha_kernel<kDN, kDR, kDV, false>), dim3((unsigned)blocks), dim3(kMThreads), 0,
                       stream, q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, sl, out, lse);
    hipLaunchKernelGGL((masked_mha_exact_kernel<kDN, kDR, kDV, false>), dim3((unsigned)blocks), dim3(kXThreads),
                       0, stream, q, k_nope, k_pe, v, bits, words, T, S, H, q_pos_offset, sl, out, lse, 1);
  }
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
