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
// MI355X design (one workgroup of 4 waves per group, one wave per SIMD):
//  * S^T = K Q^T is split by rows, O^T = V^T P^T by columns: wave w scores rows
//    32 w .. 32 w + 31 (their queries, 576 or 512 dims, sit in registers as
//    the B operand, 32 k-steps, the rest in a lane-private LDS area), runs
//    their softmax and writes their bf16 probabilities to LDS; after the
//    tile's barrier every wave multiplies all 128 rows' probabilities by its
//    own 128 value columns, so O^T (128 columns x 128 rows) fills the wave's
//    256 accumulation registers and each wave reads only a quarter of V^T.
//    The per-row softmax reference is fixed (below), so only P crosses waves;
//    the row sums meet once, at the end;
//  * iteration t runs the QK of tile t + 1 and then the PV of tile t, whose
//    MFMAs carry the softmax of tile t + 1 in pieces (masking, reference,
//    exponentials, P stores), so MFMA and VALU work overlap inside the wave;
//  * 32-slot tiles of latent rows stream through a 3-stage LDS ring by
//    asynchronous global->LDS DMA, two tiles ahead of the compute, one
//    barrier per tile.  Each wave copies one 8-row group of a tile (nine or
//    eight 128-byte blocks per row) into the XOR-swizzled 8-row-group layout
//    (common.h), so the 16-byte K reads and the transposed V reads are free of
//    bank conflicts; the copy instructions are spread between the QK MFMAs.
//    The slot indices and membership bytes of a tile arrive by their own DMA
//    four tiles ahead; per-token membership masks then come from ballots,
//    made (with the next copies' source rows) during the previous tile's PV;
//  * S^T = K Q^T and O^T = V^T P^T both run on v_mfma_f32_32x32x16_bf16 (the
//    full-rate shape); V^T comes from ds_read_b64_tr_b16, and the bf16
//    probabilities are stored in the score accumulators' own layout, which is
//    the PV B operand's (keys relabelled consistently);
//  * softmax in base 2 on raw scores (the scale folded into the exponent's
//    FMA; a negative scale negates the queries) against a per-row reference
//    fixed at the row's first valid scores, so O is written only by MFMAs.
//    Probabilities may exceed 1 by up to 2^64 (safe for bf16 P and fp32 O and
//    l); a group with a score beyond that is marked and recomputed by the
//    exact kernel (rows128_exact.hip), which ordinary inputs never reach;
//  * an FP8 latent (decoded exactly to bf16) carries a float32 scale per row:
//    the scales of a tile's slots arrive by DMA with its rows, each raw score
//    is multiplied by its row's scale before the softmax and each probability
//    by it before the PV product (l sums the unscaled probabilities);
//  * the output is staged through LDS, so that each store instruction
//    writes 256-byte row segments;
//  * longest groups (most union slots) are launched first, and the XCDs take
//    chunks of 8 consecutive groups in turn, so each gets its share of the
//    short groups at the start of a causal chunk;
//  * per-token mode (H = 128, one token per "group"): the loop ends at the
//    tile of the row's last valid slot (rows that end in -1 padding).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kRDv = 512;
constexpr int kRWaves = 4;
constexpr int kRThreads = 64 * kRWaves;
constexpr int kRKeys = 32;                          // slots per tile
constexpr int kRStages = 3;
constexpr int kRIdxBufs = 4;                        // index/membership buffers (one tile further ahead)
constexpr float kRSlack = 64.f;                     // log2 of the largest probability allowed
constexpr int kRQRegSteps = 32;                     // query k-steps kept in registers

// D: the latent width, 576 (512 + 64 rope dims) or 512 (no rope part); kScaled: the latent
// rows carry scales (kscale[scale_per_row ? x : 0] for row x)
template <int D, bool kPerToken, bool kScaled, bool kSmallKv>
__global__ __launch_bounds__(kRThreads) void rows128_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ keys, int64_t keys_ld, const int32_t* __restrict__ union_len,
    const uint8_t* __restrict__ hgmask, int T, int H, int S, int ncols, int64_t q_pos_offset,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ ginfo, const float* __restrict__ kscale, int scale_per_row,
    const int32_t* __restrict__ skip) {
  static_assert(D == 576 || D == 512, "latent widths");
  if (skip != nullptr && uniform(*skip) != 0) return;  // (another routing was chosen on the device)
  constexpr int kRGroupBytes = 8 * D * 2;           // one 8-row group (9216 / 8192)
  constexpr int kRStageBytes = 4 * kRGroupBytes;    // one 32-slot tile
  constexpr int kRCopies = kRGroupBytes / 1024;     // row copies per wave per tile (9 / 8)
  constexpr int kRQLdsSteps = D / 16 - kRQRegSteps;  // query k-steps in LDS (lane-private)
  __shared__ __align__(16) uint8_t stage[kRStages][kRStageBytes];
  // per tile and wave: lanes 0..7 = slot indices 8 w .. 8 w + 7, lanes 8, 9 = their membership bytes
  __shared__ __align__(16) uint32_t idxw[kRIdxBufs][kRWaves][64];
  __shared__ __align__(16) uint4 qlds[kRWaves][kRQLdsSteps > 0 ? kRQLdsSteps : 1][64];
  // probabilities of a tile (two buffers): wave w's lane l stores the B operand of slot step st
  // for its row block at pbuf[b][w][st][l]; every wave reads it back for row block w
  __shared__ __align__(16) bf16x8 pbuf[2][kRWaves][2][64];
  __shared__ float lsum[128];
  // kScaled: per tile and wave, lane l holds the scale of slot 8 w + l % 8
  __shared__ __align__(16) float sbuf[kScaled ? kRStages : 1][kRWaves][64];
  __shared__ int over_any;
  __shared__ int last_slot[kRWaves];  // per-token mode: each wave's last slot with a valid entry

  const int G = 128 / H;
  const int NG = (int)gridDim.x;
  // (a group's work is its union's length -- a token's, its valid slots -- which grows along
  // a causal chunk: the XCDs take chunks of 8 groups in turn, so that each gets its share of
  // the short early groups instead of one XCD getting all of them)
  const int grp = NG - 1 - xcd_chunked_block((int)blockIdx.x, NG, 8);
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;  // (wave: a scalar)
  const int hi = lane >> 5, m = lane & 31;
  const int2 span = group_span(ginfo, grp, G, T);  // (a batch's groups come from its table)
  const int t0 = uniform(span.x), ntok = uniform(span.y);
  if (ntok <= 0) return;  // (an empty group of a batch: nothing to write)
  const int r = 32 * wave + m;  // this lane's row
  const int ri = r / H;
  const int rh = r - ri * H;
  const int tok = t0 + ri;
  const bool live = ri < ntok;
  if (tid == 0) over_any = 0;  // ordered before any use by the loop's (or the final) barrier

  // a negative scale is applied as |scale| on negated queries so that the reference can be
  // taken on raw scores
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sc = fabsf(scale_log2);

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
  // validity of slot j holding latent row x (grouped: a union entry inside [0, S);
  // per-token: the selection rule)
  auto slot_ok = [&](int32_t x, int j) -> bool {
    return j < nkeys && x >= 0 && (kPerToken ? x <= pos : x < S);  // pos <= S - 1
  };
  // the row invalid slots copy (their P is 0): the list's first valid entry, a row the group
  // selects -- an unselected row (an unused slot of a paged cache) may hold anything, and 0
  // times a NaN is NaN.  With no valid entry there is nothing to attend over.  (The first
  // 64 entries are loaded in the prologue, with the queries.)
  int dummy_row = -1;
  int ntiles = 0;  // (both set in the prologue below)
  bf16x8 qreg[kRQRegSteps];  // the queries' register steps (loaded in the prologue)

  // the tokens of this wave's rows: 32 w / H and (32 w + 31) / H (two only for H = 16)
  const int ti0 = (32 * wave) / H, ti1 = (32 * wave + 31) / H;
  const bool second = ri != ti0;

  // DMA.  Index copy of tile t: lane l < 8 takes slot 8 w + l, lanes 8 and 9 the four
  // membership bytes of slots 8 w .. + 3 and 8 w + 4 .. + 7 (the others repeat slot 8 w + l % 8;
  // in per-token mode the list is the top-k row, read no further than its last column).
  // Row copies of tile t: wave w fills tile rows 8 w .. 8 w + 7 (8-row group w), blocks
  // 0 .. kRCopies - 1; lane l takes row l / 8, position l % 8.
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ swz8(crow) ^ wave;
  const uint16_t* cbase = kv + 8 * cchunk;
  const uint32_t cdst = wave * kRGroupBytes;
  const bool idx_mask_lane = !kPerToken && lane >= 8 && lane < 10;
  auto issue_idx = [&](int t) {
    const int j0 = t * kRKeys + 8 * wave;
    const int32_t* src = klist + min(j0 + (lane & 7), ncols - 1);
    if (!kPerToken)  // (a select, not a branch)
      src = idx_mask_lane ? reinterpret_cast<const int32_t*>(mlist + j0) + (lane - 8) : src;
    dma4(src, lds_addr(&idxw[t % kRIdxBufs][wave][0]));
  };
  // (kSmallKv, a latent below 2 GiB: every row offset fits 31 bits, and block c's copies take
  // the uniform base kv + 128 c plus the lane's offset, with no 64-bit address arithmetic)
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  // A tile's row copies: the source row of this lane's slot, resolved once (rows_make, which
  // also copies the slots' scales), its source and LDS destination (rows_src), then one
  // 128-byte block per copy instruction (rows_copy), so that a tile's copies can be spread
  // between MFMAs.
  struct RowSrc {
    uint32_t ofs;          // small latent: byte offset of this lane's 16 bytes of the row
    const uint16_t* src;   // otherwise: their address
    uint32_t dst;          // LDS address of the wave's 8-row group in the stage
  };
  // (the slot indices of a tile's copies: this lane's copy row, and for the scales slot
  // 8 w + l % 8 -- read from this wave's own landed words first, used later, so the LDS
  // latency can pass under MFMAs)
  auto rows_read = [&](int t) -> int2 {
    return int2{(int)idxw[t % kRIdxBufs][wave][crow], kScaled ? (int)idxw[t % kRIdxBufs][wave][lane & 7] : 0};
  };
  auto rows_src = [&](int t, uint32_t row) -> RowSrc {
    RowSrc r;
    r.dst = lds_addr(stage[t % kRStages]) + cdst;
    r.ofs = row * (2 * D) + 16 * cchunk;
    r.src = cbase + (size_t)row * D;
    return r;
  };
  auto rows_make = [&](int t, int2 xr) -> uint32_t {
    const int32_t x = xr.x;
    const bool ok = slot_ok(x, t * kRKeys + 8 * wave + crow);
    if (kScaled) {  // the scales of slots 8 w .. 8 w + 7 (lane l: slot 8 w + l % 8)
      const int32_t xs = xr.y;
      const bool oks = slot_ok(xs, t * kRKeys + 8 * wave + (lane & 7));
      dma4(kscale + (scale_per_row && oks ? xs : 0), lds_addr(&sbuf[kScaled ? t % kRStages : 0][wave][0]));
    }
    return (uint32_t)(ok ? x : dummy_row);
  };
  // (the global address carries the block offset: an instruction offset would also move the
  // LDS destination of an LDS-DMA load)
  auto rows_copy = [&](const RowSrc& r, int c) {
    if (kSmallKv)
      dma16_sbase(r.ofs, kvb + 128 * c, r.dst + 1024 * c);
    else
      dma16(r.src + 64 * c, r.dst + 1024 * c);
  };

  // K reads (A of S^T): key m, dims 16 s + 8 hi -> chunk 2 s + hi: 4 bases (s % 4) + (s / 4) KiB
  const int kx = swz8(m & 7) ^ (m >> 3) ^ hi;
  int kofs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kofs[u] = (m >> 3) * kRGroupBytes + (m & 7) * 128 + 16 * ((2 * u) ^ kx);
  // transposed V reads: key 16 st + 8 uu + 4 hi + s16 / 4, cols 32 cb + 16 (g16 % 2) + 4 (s16 % 4)
  const int g16 = lane >> 4, s16 = lane & 15;
  const int vr8 = 4 * hi + (s16 >> 2);
  const int vx = (2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ swz8(vr8);
  const int vbase = vr8 * 128 + 8 * (s16 & 1);

  // ---- per-tile pieces ------------------------------------------------------------------
  // membership of tile t's slots for this lane's row: bit kk <-> slot 4 hi + kk (kk = 8 u + jj)
  // (read: lane l takes slot l % 32's index and membership word, written by every wave's
  // copies, so after a barrier; make: the ballots)
  auto allowed_read = [&](int t) -> uint2 {
    const int sl = lane & 31;
    const uint32_t* iw = &idxw[t % kRIdxBufs][sl >> 3][0];
    return uint2{iw[sl & 7], kPerToken ? 0u : iw[8 + ((sl & 7) >> 2)]};
  };
  auto allowed_make = [&](int t, uint2 w) -> uint32_t {
    const int sl = lane & 31;
    const bool ok = slot_ok((int32_t)w.x, t * kRKeys + sl);
    uint32_t mk0, mk1;
    if (kPerToken) {
      mk0 = mk1 = (uint32_t)ballot(ok);
    } else {
      const uint32_t byte = w.y >> (8 * (sl & 3));
      mk0 = (uint32_t)ballot(ok && ((byte >> ti0) & 1u));
      mk1 = (uint32_t)ballot(ok && ((byte >> ti1) & 1u));
    }
    return (second ? mk1 : mk0) >> (4 * hi);
  };
  // kScaled: row scales of tile t's slots 8 u + 4 hi .. + 3 (score registers 4 u .. 4 u + 3)
  auto tile_scales = [&](int t, f32x4 (&ks)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ks[u] = kScaled ? *reinterpret_cast<const f32x4*>(&sbuf[kScaled ? t % kRStages : 0][u][4 * hi])
                      : f32x4{1.f, 1.f, 1.f, 1.f};
  };

  // O^T[cols 128 w + 32 cb ..][rows 32 rb ..] += V^T P^T of tile t, slot step st (slots
  // 16 st .. 16 st + 15, k-slot (hi, i) <-> slot 16 st + 8 (i / 4) + 4 hi + i % 4): the V^T
  // operand of this wave's column block cb, and the P^T operand of row block rb written by
  // wave rb (its lanes' probabilities of those slots)
  const int vcol0 = 4 * wave;  // this wave's first 32-column block
  auto vread = [&](const uint8_t* vt, int st, int cb) -> bf16x8 {
    const int cg = vcol0 + cb;
    // rows 16 st + 8 uu + vr8 are in group 2 st + uu; chunk 4 cg + c2 is in block cg / 2
    const int p0 = 16 * (vx ^ (4 * (cg & 1)) ^ (2 * st));
    const int p1 = 16 * (vx ^ (4 * (cg & 1)) ^ (2 * st + 1));
    const u16x4 lo = lds_read_tr16(vt + (2 * st) * kRGroupBytes + 1024 * (cg >> 1) + vbase + p0);
    const u16x4 up = lds_read_tr16(vt + (2 * st + 1) * kRGroupBytes + 1024 * (cg >> 1) + vbase + p1);
    return __builtin_bit_cast(bf16x8, u16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
  };

  // The first operands of tile t's PV (the V^T operands of column blocks 0 and 1 and the
  // four P^T operands of slot step 0), read during the tail of the QK before it, whose
  // last MFMAs no longer read the LDS: the PV then starts without waiting.
  bf16x8 pv_va[2], pv_pw[4];
  auto pv_pre = [&](int t) {
    const uint8_t* vt = &stage[0][0] + loop_local((t % kRStages) * kRStageBytes);
    const bf16x8* pt = &pbuf[t & 1][0][0][0] + loop_local(lane);
    pv_va[0] = vread(vt, 0, 0);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) pv_pw[rb] = pt[2 * rb * 64];
    pv_va[1] = vread(vt, 0, 1);
  };

  // S^T = K Q^T of tile t: sacc[j] = raw score(slot 8 (j / 4) + 4 hi + j % 4, row r).  The K
  // reads run kRAhead MFMAs ahead (the order is pinned: left to itself the scheduler puts
  // every read right before its MFMA and waits out its latency).  With `copy`, block c of
  // tile t + 1's row copies goes out after MFMA 4 c + 1: spread over the MFMAs, the copies do
  // not hold the wave at their issue as a burst does.  The VALU work of the next steps rides
  // here, where the MFMAs have no other company: the copy source rows of tile t + 1 (from
  // its index words `rw`, read earlier) and the membership of tile t (from `aw`) for its
  // softmax.
  auto qk = [&](int t, auto copy_tag, int2 rw, uint2 aw, uint32_t& al, int pv_t) -> f32x16 {
    constexpr bool copy = decltype(copy_tag)::value;
    RowSrc next{};
    if (copy) next = rows_src(t + 1, rows_make(t + 1, rw));
    const uint8_t* kt = &stage[0][0] + loop_local((t % kRStages) * kRStageBytes);
    // (the LDS query address is made opaque per tile, so that its reads are not hoisted)
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(&qlds[wave][0][0]) + loop_local(16 * lane);
    auto kread = [&](int st) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(kt + kofs[st & 3] + 1024 * (st >> 2));
    };
    auto qread = [&](int st) -> bf16x8 {
      return st < kRQRegSteps ? qreg[st < kRQRegSteps ? st : 0]
                              : *reinterpret_cast<const bf16x8*>(qb + 1024 * (st - kRQRegSteps));
    };
    constexpr int kRAhead = 4;
    bf16x8 kw[kRAhead], qw[kRAhead];
#pragma unroll
    for (int st = 0; st < kRAhead; ++st) {
      kw[st] = kread(st);
      qw[st] = qread(st);
    }
    f32x16 acc;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      acc = st == 0 ? mfma_qk_first(kw[0], qw[0]) : mfma_qk(kw[st % kRAhead], qw[st % kRAhead], acc);
      if (st + kRAhead < D / 16) {
        kw[st % kRAhead] = kread(st + kRAhead);
        qw[st % kRAhead] = qread(st + kRAhead);
      }
      if (copy && (st & 3) == 1 && (st >> 2) < kRCopies) rows_copy(next, st >> 2);
      if (st == 10) al = allowed_make(t, aw);  // (past the last tile: no valid slot, all masked)
      if (st == D / 16 - 4 && pv_t >= 0) pv_pre(pv_t);
    }
    __builtin_amdgcn_sched_barrier(0);
    return acc;
  };

  float m_ref = kNegInf;  // row r's reference (log2 units), equal in both halves
  float l_run = 0.f;      // this lane's partial sum (its 16 slots of every tile)
  bool over = false;
  f32x16 o[4][4];         // o[cb][rb][j] = O^T[col 128 w + 32 cb + 8 (j / 4) + 4 hi + j % 4][row 32 rb + m]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) o[cb][rb] = f32x16{};

  // The softmax of tile tn on its scores sacc, in pieces k = 0..kSmPieces - 1 that the PV
  // MFMAs of the previous tile carry: masking (and the row scales), the reference, the
  // probabilities, and their store to pbuf[tn % 2] for every wave.  The row max is needed only
  // until every row of the wave has its reference (kRef: the first tiles); after that a score
  // far above the reference shows in the probabilities' sum, which is checked at the end.
  constexpr int kSmPieces = 28;
  constexpr int kSmLag = 4;
  float sm_ml = kNegInf, sm_mr = kNegInf, sm_nm = 0.f;
  bf16x8 bop[2];
  auto sm_piece = [&](int k, int tn, f32x16& sacc, uint32_t allowed, const f32x4 (&ks)[4], auto ref_tag) {
    constexpr bool kRef = decltype(ref_tag)::value;
    if (k < 8) {  // masking of scores 2 k, 2 k + 1; the row max (raw units)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * k + jj;
        const int kk = 8 * (j >> 2) + (j & 3);
        const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)allowed, kk, 1);  // all ones if allowed
        // (a scalar copy: bit casts of vector elements misread)
        const float raw = kScaled ? sacc[j] * ks[j >> 2][j & 3] : sacc[j];
        const float val = __builtin_bit_cast(float, (sel & __builtin_bit_cast(uint32_t, raw)) | (~sel & 0xff800000u));
        sacc[j] = val;
        if (kRef) sm_ml = fmaxf(sm_ml, val);
      }
    } else if (k == 8) {  // the row max over both halves of the row
      if (!kRef) return;
      sm_ml *= sc;
      sm_mr = max_xor32(sm_ml);
    } else if (k == 9) {
      // a row's first valid scores set its reference (its O and l are still zero); both halves
      // of the row agree on it
      if (!kRef) return;
      m_ref = m_ref == kNegInf ? sm_mr : m_ref;
      over |= sm_ml > m_ref + kRSlack;
      sm_nm = m_ref == kNegInf ? 0.f : -m_ref;
      sm_ml = kNegInf;
    } else if (k < 26) {  // probability of score k - 10 (times its row scale: the PV operand)
      const int j = k - 10;
      const float p = fast_exp2(__builtin_fmaf(sacc[j], sc, sm_nm));
      l_run += p;
      asm volatile("" : "+v"(l_run));  // (the sum stays in its piece: sunk to the loop's end, the
                                       // 16 dependent adds would stall the MFMAs there)
      bop[j >> 3][j & 7] = (__bf16)(kScaled ? p * ks[j >> 2][j & 3] : p);
    } else {
      pbuf[tn & 1][wave][k - 26][lane] = bop[k - 26];
    }
  };

  // PV of tile t (V^T from stage t % 3, P^T from pbuf[t % 2]) carrying the softmax of tile
  // t + 1, whose pieces start kSmLag MFMAs in (the scores come from written-out MFMAs whose
  // latency the compiler does not see).  MFMA i: slot step st = i / 16, column block
  // cb = (i / 4) % 4, row block rb = i % 4.  A V^T operand serves four MFMAs in a row; the
  // one two column blocks on is read as it retires (two buffers, reads about five MFMAs
  // ahead, evenly spread), and the four P^T operands of a step are held through it (the next
  // step's are read as these retire).
  auto pv_sm = [&](int t, f32x16& sacc_n, uint32_t allowed_n, const f32x4 (&ks_n)[4], uint2& aw, int2& rw,
                   auto ref_tag) {
    const uint8_t* vt = &stage[0][0] + loop_local((t % kRStages) * kRStageBytes);
    const bf16x8* pt = &pbuf[t & 1][0][0][0] + loop_local(lane);
    auto pread = [&](int st, int rb) -> bf16x8 { return pt[(2 * rb + st) * 64]; };
    bf16x8 va[2] = {pv_va[0], pv_va[1]}, pw[4] = {pv_pw[0], pv_pw[1], pv_pw[2], pv_pw[3]};  // (pv_pre)
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int st = i >> 4, cb = (i >> 2) & 3, rb = i & 3;
      o[cb][rb] = mfma32x32x16(va[cb & 1], pw[rb], o[cb][rb]);
      // (the P^T read first: it is needed sooner, and LDS reads retire in order)
      if (st == 0 && cb == 3) pw[rb] = pread(1, rb);  // this P^T operand's last use in step 0
      if (rb == 3 && (i >> 2) + 2 < 8) {  // this V^T operand's last use: the one two blocks on
        const int nb = (i >> 2) + 2;
        va[cb & 1] = vread(vt, nb >> 2, nb & 3);
      }
      if (i == kSmLag) asm volatile("" : "+v"(sacc_n));  // (no read of the scores above this point)
      // the index words of the next iteration's membership (tile t + 2) and copy sources
      // (tile t + 3), made during its QK
      if (i == 8) {
        aw = allowed_read(t + 2);
        rw = rows_read(t + 3);
      }
      if (i >= kSmLag && i < kSmLag + kSmPieces) sm_piece(i - kSmLag, t + 1, sacc_n, allowed_n, ks_n, ref_tag);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the prologue ---------------------------------------------------------------------
  // The list's first entries and the slots of this lane's row copies in tiles 0 and 1 go out
  // first, then the index words of tiles 0 .. 3 and the queries; the row copies of tiles 0 and
  // 1 follow as soon as the list's head has landed, while the queries still stream in (their
  // loads, 16 rows under every quarter-wave, are limited by the address path).  (Index words
  // are copied for the tiles the list's padded length allows; past the union they are not
  // looked at.)
  const int32_t x_first = lane < ncols ? klist[lane] : -1;
  int2 xr0 = {-1, -1}, xr1 = {-1, -1};  // (rows_read's words of tiles 0 and 1, from the list)
  if (ncols > 0) {
    const int last = ncols - 1;
    xr0 = int2{klist[min(8 * wave + crow, last)], kScaled ? klist[min(8 * wave + (lane & 7), last)] : 0};
    xr1 = int2{klist[min(kRKeys + 8 * wave + crow, last)], kScaled ? klist[min(kRKeys + 8 * wave + (lane & 7), last)] : 0};
  }
  // per-token mode: the row's entries, for its last valid slot (rows end in -1 padding when a
  // token selects fewer rows than the buffer holds; the loop then stops at the last tile with
  // a valid slot).  One load per thread and 256 slots, all in flight with the queries.
  constexpr int kRScan = kPerToken ? 8 : 1;
  int32_t xs[kRScan];
  if constexpr (kPerToken) {
#pragma unroll
    for (int u = 0; u < kRScan; ++u) {
      const int j = tid + u * kRThreads;
      xs[u] = j < ncols ? klist[j] : -1;
    }
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < kRIdxBufs; ++t)
    if (t * kRKeys < ncols) issue_idx(t);
  uint4 qtail[kRQLdsSteps > 0 ? kRQLdsSteps : 1];
  {
    // queries: row r, dims 16 s + 8 hi .. + 8 (steps kRQRegSteps.. go to a lane-private LDS
    // area: the registers are needed to keep operand reads in flight).  A row past the group's
    // tokens loads the first token's row and is zeroed below: unconditional loads go out back
    // to back (a load under a branch is waited for inside it).
    const uint16_t* qrow = q + ((size_t)(live ? tok : t0) * H + rh) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 16 * s);
      if (s < kRQRegSteps)
        qreg[s] = __builtin_bit_cast(bf16x8, w);
      else
        qtail[s - kRQRegSteps] = w;
    }
  }
  asm volatile("" ::: "memory");  // (the copies below go out after the query loads)
  {
    const uint64_t b = ballot(slot_ok(x_first, lane));
    if (b != 0) dummy_row = __builtin_amdgcn_readlane(x_first, __builtin_ctzll(b));
  }
  for (int c0 = 64; dummy_row < 0 && c0 < nkeys; c0 += 64) {
    const int32_t x = c0 + lane < nkeys ? klist[c0 + lane] : -1;
    const uint64_t b = ballot(slot_ok(x, c0 + lane));
    if (b != 0) dummy_row = __builtin_amdgcn_readlane(x, __builtin_ctzll(b));
  }
  dummy_row = uniform(dummy_row);
  ntiles = uniform(dummy_row < 0 ? 0 : (nkeys + kRKeys - 1) / kRKeys);
  if (ntiles > 0) {
    const RowSrc r0 = rows_src(0, rows_make(0, xr0));
#pragma unroll
    for (int c = 0; c < kRCopies; ++c) rows_copy(r0, c);
    if (ntiles > 1) {
      const RowSrc r1 = rows_src(1, rows_make(1, xr1));
#pragma unroll
      for (int c = 0; c < kRCopies; ++c) rows_copy(r1, c);
    }
  }
  wait_vmcnt<0>();
  // (the list words and the queries are consumed here, after the wait, so the compiler counts
  // their loads as done: a load it still took for pending at the loop would put vector-memory
  // waits, which also wait for the row copies in flight, into every iteration)
  asm volatile("" : : "v"(x_first), "v"(xr0.x), "v"(xr0.y), "v"(xr1.x), "v"(xr1.y));
  if constexpr (kRQLdsSteps <= 0) {  // (else the stores of the LDS steps below consume the last loads)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : : "v"(qreg[s]));
  }
  // (the queries' sign, once they have landed: the statement orders the reads after the
  // wait.  A row past the group's tokens keeps the first token's query: its token selects
  // nothing, so every score of the row is masked, and the row is never stored.)
  if (qsign != 0) {
    auto qfix = [&](uint4 w) -> uint4 {
      asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
      w.x ^= qsign; w.y ^= qsign; w.z ^= qsign; w.w ^= qsign;
      return w;
    };
#pragma unroll
    for (int s = 0; s < kRQLdsSteps; ++s) qtail[s] = qfix(qtail[s]);
#pragma unroll
    for (int s = 0; s < kRQRegSteps; ++s) qreg[s] = __builtin_bit_cast(bf16x8, qfix(__builtin_bit_cast(uint4, qreg[s])));
  }
#pragma unroll
  for (int s = 0; s < kRQLdsSteps; ++s) qlds[wave][s][lane] = qtail[s];
  if constexpr (kPerToken) {
    int last_ok = -1;
#pragma unroll
    for (int u = 0; u < kRScan; ++u)
      if (slot_ok(xs[u], tid + u * kRThreads)) last_ok = tid + u * kRThreads;
    for (int c0 = kRScan * kRThreads; c0 < ncols; c0 += kRThreads)  // (rows past 2048 columns)
      if (c0 + tid < ncols && slot_ok(klist[c0 + tid], c0 + tid)) last_ok = c0 + tid;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) last_ok = max(last_ok, __shfl_xor(last_ok, d));
    if (lane == 0) last_slot[wave] = last_ok;
  }
  __syncthreads();  // tile 0 and the index words of tiles 0 .. 3 visible to all waves
  if constexpr (kPerToken) {
    const int last = max(max(last_slot[0], last_slot[1]), max(last_slot[2], last_slot[3]));
    ntiles = uniform(min(ntiles, (last + kRKeys) / kRKeys));  // (tiles 0 and 1 already went out)
  }

  // ---- the pipeline ---------------------------------------------------------------------
  // Iteration t: (wait + barrier) tile t + 1 and the probabilities of tile t are in LDS;
  // copy tile t + 2 into the stage of tile t - 1; QK of tile t + 1; PV of tile t carrying the
  // softmax of tile t + 1.  Stages in use: t (V), t + 1 (K), t + 2 (in flight).  A tile's
  // index words arrive four tiles ahead of its QK (issued in iteration t - 4); the words of
  // tile t + 1's membership and tile t + 2's copy sources are read during the PV of
  // iteration t - 1 and turned into masks and rows during the QK of tile t + 1.
  if (ntiles > 0) {
    f32x4 ks0[4];
    tile_scales(0, ks0);
    uint32_t al0 = 0u;
    f32x16 s0 = qk(0, std::false_type{}, int2{0, 0}, allowed_read(0), al0, -1);
    // wait states before the VALU reads the last score MFMA's results (the scores pass
    // through the statement, so no read of them can be placed above it)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0));
#pragma unroll
    for (int k = 0; k < kSmPieces; ++k) sm_piece(k, 0, s0, al0, ks0, std::true_type{});
  }
  uint2 aw = allowed_read(1);  // (words of tiles past the last are never used: no slot is valid)
  int2 rw = rows_read(2);
  auto iteration = [&](int t, auto ref_tag) {
    wait_vmcnt<0>();  // tile t + 1, the scales of tile t + 2 and the indices of tile t + 3
    __syncthreads();  // P(t) of every wave visible; stage (t + 2) % 3, pbuf (t + 1) % 2 and index
                      // buffer t % 4 free
    if (t + 4 < ntiles) issue_idx(t + 4);
    const bool copy = t + 2 < ntiles;  // (tile t + 2's blocks go out during the QK below)
    const bool more = t + 1 < ntiles;
    f32x4 ks[4];
    tile_scales(more ? t + 1 : t, ks);
    uint32_t al = 0u;  // tile t + 1's membership (0 past the last tile: all masked)
    f32x16 sn = {};
    if (copy)
      sn = qk(t + 1, std::true_type{}, rw, aw, al, t);
    else if (more)
      sn = qk(t + 1, std::false_type{}, rw, aw, al, t);
    else
      pv_pre(t);
    // (a VGPR-resident value for the softmax even past the last tile)
    pv_sm(t, sn, al, ks, aw, rw, ref_tag);
  };
  // while a row of this wave has no reference yet (normally not past tile 0), the softmax
  // takes row maxima; then the loop without them
  int t = 0;
  for (; t < ntiles && ballot(m_ref == kNegInf) != 0; ++t) iteration(t, std::true_type{});
  for (; t < ntiles; ++t) iteration(t, std::false_type{});
  // every probability is at most 2^kRSlack unless a score rose that far above its reference:
  // then this lane's sum shows it (an infinite or NaN sum as well)
  over |= !(l_run <= __builtin_ldexpf(1.f, (int)kRSlack));

  if (ballot(over) != 0 && lane == 0) over_any = 1;
  const float l = sum_xor32(l_run);
  if (hi == 0) lsum[r] = l;
  __syncthreads();
  const bool marked = over_any != 0;
  if (marked) {  // recomputed by the exact kernel
    if (live && hi == 0) lse[(size_t)tok * H + rh] = __uint_as_float(kOverflowMark);
    return;
  }
  if (live && hi == 0) lse[(size_t)tok * H + rh] = l > 0.f ? (m_ref + fast_log2(l)) * kLn2 : kNegInf;
  // The output goes out through LDS (the stages are free after the barrier above): wave w
  // turns its 128 columns of 64 rows at a time into rows of 256 contiguous bytes, so that each
  // store instruction writes four such segments.  o[cb][rb][j] = O^T[col 128 w + 32 cb +
  // 8 (j / 4) + 4 hi + j % 4][row 32 rb + m].
  constexpr int kOPitch = 272;  // bytes per staged row (256 + 16: rows start on other banks)
  static_assert(4 * 64 * kOPitch <= kRStages * kRStageBytes, "output staging fits the stages");
  uint8_t* ost = &stage[0][0] + wave * 64 * kOPitch;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int rbl = 0; rbl < 2; ++rbl) {
      const int rb = 2 * half + rbl;
      const float lr = lsum[32 * rb + m];
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const bf16x4 w = {(__bf16)(o[cb][rb][4 * jj + 0] * inv), (__bf16)(o[cb][rb][4 * jj + 1] * inv),
                            (__bf16)(o[cb][rb][4 * jj + 2] * inv), (__bf16)(o[cb][rb][4 * jj + 3] * inv)};
          *reinterpret_cast<bf16x4*>(ost + (32 * rbl + m) * kOPitch + 64 * cb + 16 * jj + 8 * hi) = w;
        }
    }
    // (a wave's LDS accesses complete in order: these reads see the writes above, and the next
    // half's writes come after the stores have taken these reads' data.)  Row r of the group
    // is token t0 + r / H, head r % H: its output row is t0 * H + r.  All 16 reads go out
    // before the first store; the rows past the group's tokens are not stored.
    uint4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = *reinterpret_cast<const uint4*>(ost + (4 * k + (lane >> 4)) * kOPitch + 16 * (lane & 15));
    uint16_t* orow = out + ((size_t)t0 * H + 64 * half + (lane >> 4)) * kRDv + 128 * wave + 8 * (lane & 15);
    const int rows_live = ntok * H - 64 * half;  // rows of this half that are stored (uniform)
    if (rows_live >= 64) {
#pragma unroll
      for (int k = 0; k < 16; ++k) *reinterpret_cast<uint4*>(orow + (size_t)(4 * k) * kRDv) = v[k];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (4 * k + (lane >> 4) < rows_live) *reinterpret_cast<uint4*>(orow + (size_t)(4 * k) * kRDv) = v[k];
    }
  }
}

template <int D, bool kPerToken, bool kScaled>
static void launch_rows128(int blocks, hipStream_t stream, const uint16_t* q, const uint16_t* kv,
                           const int32_t* keys, int64_t keys_ld, const int32_t* union_len, const uint8_t* hgmask,
                           int T, int H, int S, int ncols, int64_t q_pos_offset, float scale, uint16_t* out,
                           float* lse, const int32_t* ginfo, const float* kscale, int scale_per_row,
                           const int32_t* skip) {
  if ((int64_t)S * (2 * D) < ((int64_t)1 << 31))
    hipLaunchKernelGGL((rows128_attn_kernel<D, kPerToken, kScaled, true>), dim3(blocks), dim3(kRThreads), 0, stream,
                       q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols, q_pos_offset, scale * kLog2e, out,
                       lse, ginfo, kscale, scale_per_row, skip);
  else
    hipLaunchKernelGGL((rows128_attn_kernel<D, kPerToken, kScaled, false>), dim3(blocks), dim3(kRThreads), 0,
                       stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols, q_pos_offset,
                       scale * kLog2e, out, lse, ginfo, kscale, scale_per_row, skip);
}

template <bool kPerToken>
static void launch_rows128_any(int d_qk, int blocks, hipStream_t stream, const uint16_t* q, const uint16_t* kv,
                               const int32_t* keys, int64_t keys_ld, const int32_t* union_len,
                               const uint8_t* hgmask, int T, int H, int S, int ncols, int64_t q_pos_offset,
                               float scale, uint16_t* out, float* lse, const int32_t* ginfo, const float* kscale,
                               int scale_per_row, const int32_t* skip = nullptr) {
  if (d_qk == 512) {
    if (kscale)
      launch_rows128<512, kPerToken, true>(blocks, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                           q_pos_offset, scale, out, lse, ginfo, kscale, scale_per_row, skip);
    else
      launch_rows128<512, kPerToken, false>(blocks, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S,
                                            ncols, q_pos_offset, scale, out, lse, ginfo, kscale, scale_per_row, skip);
  } else {
    if (kscale)
      launch_rows128<576, kPerToken, true>(blocks, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S, ncols,
                                           q_pos_offset, scale, out, lse, ginfo, kscale, scale_per_row, skip);
    else
      launch_rows128<576, kPerToken, false>(blocks, stream, q, kv, keys, keys_ld, union_len, hgmask, T, H, S,
                                            ncols, q_pos_offset, scale, out, lse, ginfo, kscale, scale_per_row, skip);
  }
}

hipError_t launch_grouped_attn(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                               const int32_t* union_len, const uint8_t* head_group_mask, int T,
                               int H, int S, int union_pad, float scale, uint16_t* out, float* lse,
                               hipStream_t stream, const int32_t* group_info, int max_groups, int d_qk,
                               const float* kscale, int scale_per_row, const int32_t* skip) {
  const int G = 128 / H;
  const int NG = group_info ? max_groups : (T + G - 1) / G;
  if (NG == 0) return hipSuccess;
  launch_rows128_any<false>(d_qk, NG, stream, q, kv, union_idx, (int64_t)union_pad, union_len, head_group_mask,
                            T, H, S, union_pad, 0, scale, out, lse, group_info, kscale, scale_per_row, skip);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rows128_exact(q, kv, union_idx, (int64_t)union_pad, union_len, head_group_mask, T, H,
                              S, union_pad, 0, scale, out, lse, stream, group_info, NG, d_qk, kscale,
                              scale_per_row, skip);
}

hipError_t launch_pertoken_rows128(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                   int64_t ld, int T, int S, int cols, int64_t q_pos_offset,
                                   float scale, uint16_t* out, float* lse, hipStream_t stream, int d_qk,
                                   const float* kscale, int scale_per_row) {
  if (T == 0) return hipSuccess;
  launch_rows128_any<true>(d_qk, T, stream, q, kv, topk, ld, nullptr, nullptr, T, 128, S, cols, q_pos_offset,
                           scale, out, lse, nullptr, kscale, scale_per_row);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rows128_exact(q, kv, topk, ld, nullptr, nullptr, T, 128, S, cols, q_pos_offset, scale,
                              out, lse, stream, nullptr, T, d_qk, kscale, scale_per_row);
}

}  // namespace dsa
