// Per-token sparse MQA prefill over a bf16 latent of 576 dims (512 + 64 rope) or
// 512 dims (no rope part).
//
// Definition ("[Perf][GLM-5.3-Flash] Dense/masked-MHA sparse prefill for the
// NoPE (256, 0, 256) layout ...", Purpose section; "[Perf][DSA] Grouped sparse
// prefill ...", commit message): every query token attends, for each of its H
// heads, over the latent rows of its own top-k selection; scores use every dim
// of the row, values are its first 512 dims; the result is out [T, H, 512]
// (bf16) and LSE [T, H] (fp32, natural log).  The pages find this kernel bound
// by the KV gather (2048 rows x 1152 B per token for the 576-wide latent).
//
// MI355X design: one wave per (token, 16-head block), one wave per workgroup
// (no barriers), one wave per SIMD.  Two kernels share the arithmetic:
//  * sorted walk (caches of up to 2^20 rows, rows of any width with at most
//    2048 valid entries): the wave first sorts its token's valid entries in
//    LDS, so that the concurrent tokens of a range, which select nearly the
//    same rows, walk them in the same order and find them in L2.
//    Rows then stream 16 at a time into two LDS tiles (18 KiB at 576 dims) by asynchronous
//    global->LDS copies, one step ahead of the compute (each copy instruction
//    covers one 128-byte line of 8 rows, so a quarter-wave touches two cache
//    lines); the 16 heads' queries stay in registers;
//  * register ring (any size; also taken inside the sorted kernel when a
//    token has more than 2048 valid entries): rows are loaded with the same
//    coalesced pattern
//    into two register buffers, each refilled two steps ahead as soon as it
//    has been written to an LDS tile of 16 rows; the queries sit in a lane-private
//    LDS area;
//  * both: invalid entries (-1, past the row, beyond the token's position)
//    fetch the token's first valid row and are masked (P = 0); a row the
//    token selects holds real data, where an unselected one (an unused slot
//    of a paged cache) may hold anything, and 0 times a NaN would be NaN.  A
//    token with no valid entry writes zeros and -inf at once.  The tiles are XOR-swizzled,
//    free of bank conflicts for the writes, the 16-byte K reads and the
//    transposed V reads.  S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16 (one
//    accumulation chain in the sorted walk, three in the ring kernel, whose
//    exact routine the sorted walk shares); O^T = V^T P^T runs on
//    v_mfma_f32_16x16x16_bf16 with V^T from ds_read_b64_tr_b16 and the
//    probabilities straight from the score accumulators as the B operand.
//    Operand reads run several MFMAs ahead (the order is pinned: left to
//    itself the scheduler puts every read right before its MFMA);
//  * fp32 softmax in base 2 on raw scores (the scale is folded into the
//    exponent's FMA; a negative scale negates the queries) against a per-head
//    reference fixed at the head's first valid scores, so O is only ever
//    written by MFMAs and stays in the accumulation registers; each lane keeps
//    its own partial sum, so the common path has no cross-lane reduction.
//    Probabilities may exceed 1 by up to 2^64 (safe for bf16 P and fp32 O and
//    l); a token with a score beyond that is recomputed by an exact two-pass
//    routine (max first), which is not met with ordinary inputs;
//  * an FP8 latent (decoded exactly to bf16) carries a float32 scale per row:
//    each raw score is multiplied by its row's scale before the softmax and
//    each probability by it before the PV product (l sums the unscaled
//    probabilities).  The LDS is fully used by the tiles and the sorted list,
//    so the scales of a step's 16 rows come by scalar loads (their row indices
//    read out of the lanes), issued a step ahead of their use;
//  * token order is reversed (long causal rows first) and block ids are
//    remapped so each XCD runs chunks of 16 consecutive tokens, the XCDs taking
//    the chunks in turn: neighbouring tokens, which share most of their rows,
//    hit the same L2, and every XCD gets its share of the short early rows.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kDv = 512;                    // values: the first 512 dims of a latent row
constexpr int kPKeys = 16;                  // keys per step
constexpr float kPSlack = 64.f;             // log2 of the largest probability allowed

// Row geometry of latent width D: 576 (512 + 64 rope dims) or 512 (no rope part).
template <int D>
struct Lat {
  static_assert(D == 576 || D == 512, "latent widths");
  static constexpr int loads = D / 32;               // 16-byte chunks per lane per step (18 / 16)
  static constexpr int lines = D * 2 / 128;          // 128-byte lines per latent row (9 / 8)
  static constexpr int row_bytes = D * 2;            // 1152 / 1024
  static constexpr int group_bytes = 8 * row_bytes;  // one 8-row group of a sorted-walk tile
};
constexpr int kDqkMax = 576;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
// (a native vector: row chunks loaded into HIP's uint4 struct through a byte pointer
// become memcpys into a stack array that is never promoted to registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(s16x4_t a, s16x4_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// LDS of the (single-wave) workgroup, sized for the wider latent: the rows of the current
// step -- chunk c (16 B, 0..D/8-1) of row r (0..15) at r * 2D + 16 (c ^ tswz(r)); the XOR
// stays inside a 128-byte line -- and the queries, lane-private: lane l's chunk s at
// pt_q[s][l].
__shared__ __align__(16) uint8_t pt_tile[kPKeys * Lat<kDqkMax>::row_bytes];
__shared__ __align__(16) uint4 pt_q[Lat<kDqkMax>::loads][64];
// sorted mode: the token's valid entries in ascending order, each as its low 16 bits (the
// 65536-row window of list index i is the number of window starts at or below i; the starts
// travel in a register, one window per lane)
constexpr int kPSortMax = 2048;
constexpr int kPSortRows = 1 << 20;  // caches up to this many rows (16 windows; row offsets below 2^31)
__shared__ __align__(16) uint16_t pt_sorted[kPSortMax];

// the list entry at index i (below the list length), with its window restored
__device__ __forceinline__ int pt_list_entry(int i, int wstart) {
  int w = 0;
  for (int u = 1; u < 16; ++u) w += __builtin_amdgcn_readlane(wstart, u) <= i ? 1 : 0;
  return (int)pt_sorted[i] | (w << 16);
}

__device__ __forceinline__ int tswz(int r) { return (2 * (r >> 1) + (r >> 3)) & 7; }

// Row scales of a step's 16 keys.  Lane l holds the row indices of keys l / 8 (rows.x) and
// 8 + l / 8 (rows.y); the scales come by uniform scalar loads (no LDS, no vector-memory
// count), and each lane then keeps those of its keys 4 g .. 4 g + 3.
struct StepScales {
  float v[16];
};
__device__ __forceinline__ StepScales step_scales_load(const float* kscale, int per_row, int2 rows) {
  StepScales st;
  const_i32* sp = uniform_const(reinterpret_cast<const int32_t*>(kscale));
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int x0 = __builtin_amdgcn_readlane(rows.x, 8 * r);
    const int x1 = __builtin_amdgcn_readlane(rows.y, 8 * r);
    st.v[r] = __int_as_float(sp[per_row ? x0 : 0]);
    st.v[8 + r] = __int_as_float(sp[per_row ? x1 : 0]);
  }
  return st;
}
__device__ __forceinline__ f32x4 step_scales_mine(const StepScales& st, int g) {
  f32x4 r;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    r[jj] = g == 0 ? st.v[jj] : g == 1 ? st.v[4 + jj] : g == 2 ? st.v[8 + jj] : st.v[12 + jj];
  return r;
}

// What one wave needs to walk its token's row.
struct PtCtx {
  const int32_t* trow;  // the token's top-k row
  const uint8_t* kvb;   // latent base + 16 (lane % 8): this lane's 16 bytes of each line
  int cols, pos, lane, g, n;
  int dummy;            // the row invalid entries fetch: the token's first valid entry
  int er;               // the rows this lane loads: er and 8 + er of each step
  float sc;             // |scale| * log2(e)
  int wofs[2];          // tile store offsets (rows er, 8 + er; + 128 per line)
  int kofs[2];          // K read offsets (row n, chunk 4 s + g: per s % 2; + 128 (s / 2))
  int rofs[4];          // transposed V read offsets (per column block cb % 4; + 128 (cb / 4))
};

// The first entry x of a top-k row with 0 <= x <= pos (pos <= S - 1), or -1 (uniform).
__device__ __forceinline__ int pt_first_valid(const int32_t* trow, int cols, int pos, int lane) {
  for (int c0 = 0; c0 < cols; c0 += 64) {
    const int x = c0 + lane < cols ? trow[c0 + lane] : -1;
    const uint64_t b = ballot(x >= 0 && x <= pos);
    if (b != 0) return uniform(__builtin_amdgcn_readlane(x, __builtin_ctzll(b)));
  }
  return -1;
}

// The per-wave context for token `token` (built in registers; the exact routine rebuilds
// it from the same scalars rather than taking it by reference, which would put it in
// scratch memory for the whole kernel).
template <int D>
__device__ __forceinline__ PtCtx pt_context(const uint16_t* kv, const int32_t* topk, int64_t ld, int S,
                                            int cols, int64_t q_pos_offset, float scale_log2, int token) {
  PtCtx c;
  c.lane = threadIdx.x;
  c.g = c.lane >> 4;
  c.n = c.lane & 15;
  int64_t pos64 = q_pos_offset + token;
  if (pos64 > S - 1) pos64 = S - 1;  // positions beyond S - 1 cannot be selected
  c.pos = uniform((int)pos64);
  c.cols = cols;
  c.trow = topk + (size_t)token * ld;
  c.er = c.lane >> 3;
  c.kvb = reinterpret_cast<const uint8_t*>(kv) + 16 * (c.lane & 7);
  c.sc = fabsf(scale_log2);
  // LDS tile offsets.  Stores: lane l writes 16 bytes l % 8 of each line of rows er and
  // 8 + er.  K reads: lane (g, n) reads row n, chunk 4 s + g.  Transposed reads for O^T
  // block cb (cols 16 cb .. + 15): lane (g, i) of a 16-lane group addresses row 4 g + i / 4,
  // cols 16 cb + 4 (i % 4) .. + 3 (chunk 2 cb + (i % 4) / 2, half i % 2), so that output
  // lane (g, n) receives V[key 4 g + jj][col 16 cb + n], jj = 0..3.
  {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + c.er;
      c.wofs[h] = r * Lat<D>::row_bytes + 16 * ((c.lane & 7) ^ tswz(r));
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) c.kofs[p] = c.n * Lat<D>::row_bytes + 16 * ((4 * p + c.g) ^ tswz(c.n));
    const int rr = 4 * c.g + (c.n >> 2);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      c.rofs[u] = rr * Lat<D>::row_bytes + 8 * (c.n & 1) + 16 * ((2 * u + ((c.n & 3) >> 1)) ^ tswz(rr));
  }

  return c;
}

// this lane's entries of step j: rows er and 8 + er (clamped into the list: the top-k row,
// or in sorted mode the sorted valid entries, c.cols of them)
template <bool kSorted>
__device__ __forceinline__ int2 pt_entries(const PtCtx& c, int j, int wstart = 0) {
  const int i0 = min(kPKeys * j + c.er, c.cols - 1), i1 = min(kPKeys * j + 8 + c.er, c.cols - 1);
  if (kSorted) return int2{pt_list_entry(i0, wstart), pt_list_entry(i1, wstart)};
  return int2{c.trow[i0], c.trow[i1]};
}

// start the loads of step j's rows into `buf` (buf[k]: line k of row er, buf[9 + k]: of row
// 8 + er); returns the validity bits of the step's 16 keys (key r <-> bit r)
template <int D>
__device__ __forceinline__ uint32_t pt_issue(const PtCtx& c, int2 e, int j, u32x4 (&buf)[Lat<D>::loads],
                                             int2& rows) {
  const bool ok0 = kPKeys * j + c.er < c.cols && e.x >= 0 && e.x <= c.pos;
  const bool ok1 = kPKeys * j + 8 + c.er < c.cols && e.y >= 0 && e.y <= c.pos;
  rows = int2{ok0 ? e.x : c.dummy, ok1 ? e.y : c.dummy};  // (the rows the loads fetch)
  const uint8_t* src0 = c.kvb + (size_t)rows.x * Lat<D>::row_bytes;
  const uint8_t* src1 = c.kvb + (size_t)rows.y * Lat<D>::row_bytes;
#pragma unroll
  for (int k = 0; k < Lat<D>::lines; ++k) {
    buf[k] = *reinterpret_cast<const u32x4*>(src0 + 128 * k);
    buf[Lat<D>::lines + k] = *reinterpret_cast<const u32x4*>(src1 + 128 * k);
  }
  // key r's validity is that of lanes 8 (r % 8) .. + 7 (bits 8 (r % 8) of the ballots)
  const uint64_t b0 = ballot(ok0), b1 = ballot(ok1);
  uint32_t v = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) v |= (uint32_t)((b0 >> (8 * r)) & 1u) << r | (uint32_t)((b1 >> (8 * r)) & 1u) << (8 + r);
  return v;
}

template <int D>
__device__ __forceinline__ void pt_store(const PtCtx& c, const u32x4 (&buf)[Lat<D>::loads]) {
#pragma unroll
  for (int k = 0; k < Lat<D>::lines; ++k) {
    *reinterpret_cast<u32x4*>(pt_tile + c.wofs[0] + 128 * k) = buf[k];
    *reinterpret_cast<u32x4*>(pt_tile + c.wofs[1] + 128 * k) = buf[Lat<D>::lines + k];
  }
}

// S^T[key 4 g + jj][head n] (raw) of the tile's rows, in three independent chains.  The K
// and query reads run kPQAhead MFMAs ahead (the order is pinned: left to itself the
// scheduler puts every read right before its MFMA and waits out its latency).
constexpr int kPQAhead = 4;
template <int D>
__device__ __forceinline__ f32x4 pt_qk(const PtCtx& c) {
  // (the query address is made opaque: hoisted out of a loop, the 18 reads would pin 72
  // registers for the whole token)
  const uint8_t* qb = reinterpret_cast<const uint8_t*>(&pt_q[0][0]) + loop_local(16 * c.lane);
  auto kread = [&](int s) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(pt_tile + c.kofs[s & 1] + 128 * (s >> 1));
  };
  auto qread = [&](int s) -> bf16x8 { return *reinterpret_cast<const bf16x8*>(qb + 1024 * s); };
  bf16x8 kw[kPQAhead], qw[kPQAhead];
#pragma unroll
  for (int s = 0; s < kPQAhead; ++s) {
    kw[s] = kread(s);
    qw[s] = qread(s);
  }
  f32x4 acc[3] = {};
#pragma unroll
  for (int s = 0; s < Lat<D>::loads; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    acc[s % 3] = mfma16x16x32(kw[s % kPQAhead], qw[s % kPQAhead], acc[s % 3]);
    if (s + kPQAhead < Lat<D>::loads) {
      kw[s % kPQAhead] = kread(s + kPQAhead);
      qw[s % kPQAhead] = qread(s + kPQAhead);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  return acc[0] + acc[1] + acc[2];
}

// invalid keys -> -inf (kScaled: valid scores times their row scales ks); returns the max of
// this lane's 4 scores
template <bool kScaled>
__device__ __forceinline__ float pt_mask(const PtCtx& c, const f32x4& sacc, uint32_t vbits, float (&sv)[4],
                                         f32x4 ks) {
  const uint32_t mine = vbits >> (4 * c.g);
  float mt = kNegInf;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)mine, jj, 1);  // all ones if valid
    // (a scalar copy: bit casts of vector elements misread)
    const float raw = kScaled ? sacc[jj] * ks[jj] : sacc[jj];
    sv[jj] = __builtin_bit_cast(float, (sel & __builtin_bit_cast(uint32_t, raw)) | (~sel & 0xff800000u));
    mt = fmaxf(mt, sv[jj]);
  }
  return mt;
}

// P = 2^(s sc - m) (bf16, as the B operand P^T[key 4 g + jj][head n]; kScaled: times the
// key's row scale); adds the unscaled P to l
template <bool kScaled>
__device__ __forceinline__ s16x4_t pt_probs(const PtCtx& c, const float (&sv)[4], float m, float& l, f32x4 ks) {
  const float nm = m == kNegInf ? 0.f : -m;
  bf16x4 pb;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float p = fast_exp2(__builtin_fmaf(sv[jj], c.sc, nm));
    l += p;
    pb[jj] = (__bf16)(kScaled ? p * ks[jj] : p);
  }
  return __builtin_bit_cast(s16x4_t, pb);
}

// O^T[col 16 cb + 4 g + jj][head n] += V^T P^T.  The transposed reads run kPVAhead MFMAs
// ahead (order pinned as in pt_qk).
constexpr int kPVAhead = 6;
__device__ __forceinline__ void pt_pv(const PtCtx& c, s16x4_t bop, f32x4 (&o)[kDv / 16]) {
  auto vread = [&](int cb) -> u16x4 { return lds_read_tr16(pt_tile + c.rofs[cb & 3] + 128 * (cb >> 2)); };
  u16x4 vw[kPVAhead];
#pragma unroll
  for (int i = 0; i < kPVAhead; ++i) vw[i] = vread(i);
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) {
    __builtin_amdgcn_sched_barrier(0);
    o[cb] = mfma16x16x16(__builtin_bit_cast(s16x4_t, vw[cb % kPVAhead]), bop, o[cb]);
    if (cb + kPVAhead < kDv / 16) vw[cb % kPVAhead] = vread(cb + kPVAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void pt_write(int g, const f32x4 (&o)[kDv / 16], float l_part, float m,
                                         uint16_t* orow, float* lse_at) {
  const float l = sum_over_rowgroups(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) {
    const bf16x4 w = {(__bf16)(o[cb][0] * inv), (__bf16)(o[cb][1] * inv), (__bf16)(o[cb][2] * inv),
                      (__bf16)(o[cb][3] * inv)};
    *reinterpret_cast<bf16x4*>(orow + 16 * cb) = w;
  }
  if (g == 0) *lse_at = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
}

// Exact two-pass routine: head n's max over the whole row first, then the softmax
// against it (no probability exceeds 1).  Both passes share pt_qk / pt_mask with the main
// loop, so their scores are bit-identical.
template <int D, bool kSorted, bool kScaled>
__device__ __noinline__ void pt_exact(const uint16_t* kv, const int32_t* topk, int64_t ld, int S, int cols,
                                     int64_t q_pos_offset, float scale_log2, int token, uint16_t* orow,
                                     float* lse_at, int wstart, const float* kscale, int per_row, int dummy) {
  PtCtx c = pt_context<D>(kv, topk, ld, S, cols, q_pos_offset, scale_log2, token);
  c.dummy = dummy;
  const int nsteps = (c.cols + kPKeys - 1) / kPKeys;
  float m = kNegInf;
  for (int j = 0; j < nsteps; ++j) {
    u32x4 buf[Lat<D>::loads];
    int2 rows;
    const uint32_t vbits = pt_issue<D>(c, pt_entries<kSorted>(c, j, wstart), j, buf, rows);
    f32x4 ks = {1.f, 1.f, 1.f, 1.f};
    if (kScaled) ks = step_scales_mine(step_scales_load(kscale, per_row, rows), c.g);
    pt_store<D>(c, buf);
    float sv[4];
    m = fmaxf(m, pt_mask<kScaled>(c, pt_qk<D>(c), vbits, sv, ks));
  }
  m = max_over_rowgroups(m) * c.sc;
  float l = 0.f;
  f32x4 o[kDv / 16];
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nsteps; ++j) {
    u32x4 buf[Lat<D>::loads];
    int2 rows;
    const uint32_t vbits = pt_issue<D>(c, pt_entries<kSorted>(c, j, wstart), j, buf, rows);
    f32x4 ks = {1.f, 1.f, 1.f, 1.f};
    if (kScaled) ks = step_scales_mine(step_scales_load(kscale, per_row, rows), c.g);
    pt_store<D>(c, buf);
    float sv[4];
    pt_mask<kScaled>(c, pt_qk<D>(c), vbits, sv, ks);
    pt_pv(c, pt_probs<kScaled>(c, sv, m, l, ks), o);
  }
  pt_write(c.g, o, l, m, orow, lse_at);
}

// The register-ring walk of one (token, 16-head block): the whole work of the ring kernel,
// and the sorted kernel's path for a token with more valid entries than its list holds.
// (Scalars only in the signature: a struct passed to a non-inlined function would live in
// scratch memory.)
template <int D, bool kScaled>
__device__ __noinline__ void pt_ring_token(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                           const int32_t* __restrict__ topk, int64_t ld, int H, int S, int cols,
                                           int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out,
                                           float* __restrict__ lse, int token, int hb, const float* kscale,
                                           int per_row) {
  PtCtx c = pt_context<D>(kv, topk, ld, S, cols, q_pos_offset, scale_log2, token);
  c.dummy = pt_first_valid(c.trow, c.cols, c.pos, c.lane);

  // queries of head n, dims 32 s + 8 g .. + 8 (the B operand of S^T = K Q^T); a negative
  // scale is applied as |scale| on negated queries so the max can be taken on raw scores
  {
    const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
    const uint16_t* qrow = q + ((size_t)token * H + hb * 16 + c.n) * D + 8 * c.g;
#pragma unroll
    for (int s = 0; s < Lat<D>::loads; ++s) {
      uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * s);
      w.x ^= qsign; w.y ^= qsign; w.z ^= qsign; w.w ^= qsign;
      pt_q[s][c.lane] = w;
    }
  }
  uint16_t* orow = out + ((size_t)token * H + hb * 16 + c.n) * kDv + 4 * c.g;
  float* lse_at = lse + (size_t)token * H + hb * 16 + c.n;
  if (c.dummy < 0) {  // nothing selected: zero output, LSE -inf
    const f32x4 z[kDv / 16] = {};
    pt_write(c.g, z, 0.f, kNegInf, orow, lse_at);
    return;
  }

  // The main loop runs an even number of steps (an odd count gets one all-masked step,
  // which adds nothing), so that it has a single exit.  Step j lives in register buffer
  // j % 2; once its rows are stored to the LDS tile the buffer receives step j + 2's rows,
  // in flight during the rest of step j and all of step j + 1.  The entries of step j + 3
  // are read before step j + 2's loads, so that waiting for an entry never waits for rows
  // issued after it.
  const int nsteps = (c.cols + kPKeys - 1) / kPKeys;
  const int nsteps2 = nsteps + (nsteps & 1);
  float m_ref = kNegInf;  // head n's reference (log2 units); equal in the 4 lane groups
  float l_run = 0.f;      // this lane's partial sum (keys 4 g .. 4 g + 3 of every step)
  f32x4 o[kDv / 16];
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ra[Lat<D>::loads], rb[Lat<D>::loads];
  uint32_t va = 0, vb = 0;
  f32x4 sa = {1.f, 1.f, 1.f, 1.f}, sb = sa;  // kScaled: this lane's row scales of the buffered steps
  int2 e_next = {0, 0};  // entries of the step whose loads start next
  {  // issue order as in the loop (entries, rows, entries, rows), pinned by scheduling
     // barriers: the wait counts at the loop head merge this order with the loop's
    const int2 e0 = pt_entries<false>(c, 0);
    const int2 e1 = pt_entries<false>(c, 1);
    int2 rows0, rows1;
    __builtin_amdgcn_sched_barrier(0);
    va = pt_issue<D>(c, e0, 0, ra, rows0);
    __builtin_amdgcn_sched_barrier(0);
    e_next = pt_entries<false>(c, 2);
    __builtin_amdgcn_sched_barrier(0);
    vb = pt_issue<D>(c, e1, 1, rb, rows1);
    __builtin_amdgcn_sched_barrier(0);
    if (kScaled) {
      sa = step_scales_mine(step_scales_load(kscale, per_row, rows0), c.g);
      sb = step_scales_mine(step_scales_load(kscale, per_row, rows1), c.g);
    }
  }
  // one step; `over` becomes true when a score exceeds the reference by more than the
  // slack (the loop still runs to its end, and its result is then discarded)
  bool over = false;
  auto step = [&](int j, u32x4 (&buf)[Lat<D>::loads], uint32_t& vbuf, f32x4& sbuf) {
    pt_store<D>(c, buf);
    const uint32_t vbits = vbuf;
    const f32x4 ks = sbuf;
    int2 rows;
    // the refill must not be scheduled above the stores that read the buffer
    __builtin_amdgcn_sched_barrier(0);
    {  // (unconditional: past the row the loads are masked dummies, and the wait
       // counts stay exact only on a branch-free path)
      const int2 e = e_next;
      e_next = pt_entries<false>(c, j + 3);
      __builtin_amdgcn_sched_barrier(0);
      vbuf = pt_issue<D>(c, e, j + 2, buf, rows);
    }
    __builtin_amdgcn_sched_barrier(0);
    const f32x4 sacc = pt_qk<D>(c);
    // kScaled: step j + 2's scales, loaded under this step's softmax and selected after its PV
    StepScales st;
    if (kScaled) st = step_scales_load(kscale, per_row, rows);
    float sv[4];
    const float mt = pt_mask<kScaled>(c, sacc, vbits, sv, ks) * c.sc;
    // a head's first valid scores set its reference (its O and l are still zero)
    if (ballot(m_ref == kNegInf && mt != kNegInf) != 0) {
      const float mh = max_over_rowgroups(mt);
      m_ref = m_ref == kNegInf ? mh : m_ref;
    }
    over |= ballot(mt > m_ref + kPSlack) != 0;
    pt_pv(c, pt_probs<kScaled>(c, sv, m_ref, l_run, ks), o);
    if (kScaled) sbuf = step_scales_mine(st, c.g);
  };
  for (int j = 0; j < nsteps2; j += 2) {
    step(j, ra, va, sa);
    step(j + 1, rb, vb, sb);
  }
  if (over) {
    pt_exact<D, false, kScaled>(kv, topk, ld, S, cols, q_pos_offset, scale_log2, token, orow, lse_at, 0, kscale,
                                per_row, c.dummy);
    return;
  }
  pt_write(c.g, o, l_run, m_ref, orow, lse_at);
}

template <int D, bool kScaled>
__global__ __launch_bounds__(64) void pertoken_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, int64_t ld, int T, int H, int S, int cols,
    int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ kscale, int per_row, const int32_t* __restrict__ skip) {
  if (skip != nullptr && uniform(*skip) != 0) return;  // (another routing was chosen on the device)
  const int nb = H >> 4;
  const int item = xcd_chunked_block((int)blockIdx.x, (int)gridDim.x, 16 * (H >> 4));  // (16 tokens)
  const int tq = item / nb;
  pt_ring_token<D, kScaled>(q, kv, topk, ld, H, S, cols, q_pos_offset, scale_log2, out, lse, T - 1 - tq,
                            item - tq * nb, kscale, per_row);
}

// ---------------------------------------------------------------------------
// Sorted-walk kernel (caches of up to kPSortRows rows; a token with more than kPSortMax
// valid entries takes the register-ring walk instead).
//
// The wave first sorts its token's valid entries (0 <= x <= position) into pt_sorted:
// a bitmap of the positions in the LDS tile, the count of set bits below each bitmap word,
// and each entry stored at its rank, one 131072-position chunk at a time.  Tokens of a range
// select nearly the same rows, so walking them in the same order lets concurrent tokens find
// each other's rows in L2.  (Repeated entries collapse to one.)  Rows then stream into two
// LDS tiles of 16 rows (18 KiB at D = 576) by asynchronous global->LDS copies (one step
// ahead; no register ring and no LDS store instructions), in the 8-row-group layout of
// common.h: 16-byte chunk k of tile row r at
// 16 D (r / 8) + 1024 (k / 8) + 128 (r % 8) + 16 ((k % 8) ^ swz8(r % 8) ^ (r / 8)).
// The queries stay in registers.  The exact fallback reuses the register-ring
// routines (the second tile is the query area there).
// ---------------------------------------------------------------------------

// Sorts the token's valid entries (0 <= x <= pos) into pt_sorted and returns how many there
// are (repeated entries collapse to one; past kPSortMax the count goes on but nothing more is
// stored).  Positions are taken in chunks of 131072.  For each chunk: a bitmap of its positions
// in the tile (16 KiB at most); for every bitmap word, the number of set bits below it (in the
// query area); then every entry writes itself at its rank, the set bits below it.  The work
// follows the entries, wherever in [0, pos] they lie.  Each 65536-position window's first list
// index goes to lane w of `wstart` (lanes of windows past the last position hold the count).
constexpr int kPSortRegs = 5;  // 8-entry batches of the row held in registers (2560 columns)

__device__ __forceinline__ int pt_sort(const int32_t* trow, int cols, int pos, int lane, int& wstart) {
  uint32_t* bm = reinterpret_cast<uint32_t*>(pt_tile);
  uint32_t* below = reinterpret_cast<uint32_t*>(&pt_q[0][0]);  // per word: list index of its first bit
  // the row's first 2560 entries in one round trip (columns past them are read once per pass)
  int32_t xr[kPSortRegs * 8];
#pragma unroll
  for (int u = 0; u < kPSortRegs * 8; ++u) xr[u] = lane + 64 * u < cols ? trow[lane + 64 * u] : -1;
  int total = 0;
  wstart = 0;
  const int nchunks = uniform((pos >> 17) + 1);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int lo = ch << 17;
    const int hi = min(pos, lo + (1 << 17) - 1);  // inclusive
    const int nw = ((hi - lo) >> 5) + 1;          // bitmap words of the chunk
    for (int w = lane; w < nw; w += 64) bm[w] = 0u;
    __syncthreads();  // (one wave: orders the LDS accesses for the compiler)
    auto mark = [&](int x) {
      if (x >= lo && x <= hi) atomicOr(&bm[(x - lo) >> 5], 1u << (x & 31));
    };
#pragma unroll
    for (int u = 0; u < kPSortRegs * 8; ++u) mark(xr[u]);
    for (int c = kPSortRegs * 512 + lane; c < cols; c += 64) mark(trow[c]);
    __syncthreads();
    // lane l owns words l * wpl .. + wpl - 1; the odd stride puts the 64 lanes of each read
    // in 64 different banks
    const int wpl = ((nw + 63) >> 6) | 1;
    const int w0 = lane * wpl, w1 = min(nw, w0 + wpl);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
    int ctot;
    int run = total + wave_incl_scan(cnt, ctot) - cnt;
    for (int w = w0; w < w1; ++w) {
      below[w] = (uint32_t)run;
      run += __popc(bm[w]);
    }
    __syncthreads();
    auto place = [&](int x) {
      if (x >= lo && x <= hi) {
        const int w = (x - lo) >> 5;
        const int at = (int)below[w] + __popc(bm[w] & ((1u << (x & 31)) - 1u));
        if (at < kPSortMax) pt_sorted[at] = (uint16_t)x;  // the low 16 bits (lo % 65536 = 0)
      }
    };
#pragma unroll
    for (int u = 0; u < kPSortRegs * 8; ++u) place(xr[u]);
    for (int c = kPSortRegs * 512 + lane; c < cols; c += 64) place(trow[c]);
    ctot = uniform(ctot);
    if (lane == 2 * ch) wstart = total;
    if (lane == 2 * ch + 1) wstart = nw > 2048 ? (int)below[2048] : total + ctot;
    total += ctot;
    __syncthreads();  // the bitmap is cleared again, or the tile rewritten, from here on
  }
  if (lane >= 2 * nchunks) wstart = total;
  return total;
}

struct PdCtx {
  int cols, pos, lane, g, n, er;
  int dummy;    // the row copies past the list fetch: the list's first entry
  int wstart;   // lane w: list index of window w's first entry (windows of 65536 positions)
  bool multi;   // the list spans more than one window
  float sc;
  int dofs[2];  // this lane's 16 bytes of each 128-byte line, for rows er (h = 0) and 8 + er (h = 1)
  int kofs[2];  // K read offsets (row n, chunk 4 s + g: per s % 2; + 1024 (s / 2))
  int rofs[4];  // transposed V read offsets (per column block cb % 4; + 1024 (cb / 4))
};

template <int D>
__device__ __forceinline__ PdCtx pd_context(int pos, int cols, float scale_log2, int wstart) {
  PdCtx c;
  c.wstart = wstart;
  c.dummy = uniform(pt_list_entry(0, wstart));
  c.multi = pos >= 65536;
  c.lane = threadIdx.x;
  c.g = c.lane >> 4;
  c.n = c.lane & 15;
  c.er = c.lane >> 3;
  c.pos = pos;
  c.cols = cols;
  c.sc = fabsf(scale_log2);
  // copies: lane l fills position l % 8 of row l / 8 of a group's 1 KiB block, i.e. it
  // fetches chunk (l % 8) ^ swz8(l / 8) ^ h of the block's 128-byte line
#pragma unroll
  for (int h = 0; h < 2; ++h) c.dofs[h] = 16 * ((c.lane & 7) ^ swz8(c.er) ^ h);
  // K reads: lane (g, n) reads row n, chunk 4 s + g
  const int kg = c.n >> 3, k8 = c.n & 7;
#pragma unroll
  for (int p = 0; p < 2; ++p) c.kofs[p] = kg * Lat<D>::group_bytes + 128 * k8 + 16 * ((4 * p + c.g) ^ swz8(k8) ^ kg);
  // transposed reads for block cb: lane (g, i) addresses row 4 g + i / 4, cols 16 cb + 4 (i % 4)
  // .. + 3 (chunk 2 cb + (i % 4) / 2, half i % 2): output lane (g, n) receives
  // V[key 4 g + jj][col 16 cb + n]
  const int rr = 4 * c.g + (c.n >> 2), rg = rr >> 3, r8 = rr & 7;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    c.rofs[u] = rg * Lat<D>::group_bytes + 128 * r8 + 16 * ((2 * u + ((c.n & 3) >> 1)) ^ swz8(r8) ^ rg) + 8 * (c.n & 1);
  return c;
}

// validity bits of step j's 16 keys (key r <-> bit r): the sorted list holds only valid
// entries, so key r is valid iff 16 j + r < n (list length n)
__device__ __forceinline__ uint32_t pd_valid(const PdCtx& c, int j) {
  const int left = c.cols - kPKeys * j;
  return left >= kPKeys ? 0xffffu : (left <= 0 ? 0u : (1u << left) - 1u);
}

// start the copies of step j's rows into the tile at LDS address `tile`; returns the
// validity bits of the step's 16 keys (past the list the copies fetch the token's own row)
// (positions are below 2^20 here, so a row's byte offset fits 31 bits; line k's copies take
// the base kvb + 128 k and the lane's row offset)
template <int D>
__device__ __forceinline__ uint32_t pd_issue(const PdCtx& c, const uint8_t* kvb, int2 e, int j, uint32_t tile) {
  const bool ok0 = kPKeys * j + c.er < c.cols;
  const bool ok1 = kPKeys * j + 8 + c.er < c.cols;
  const uint32_t off0 = (uint32_t)(ok0 ? e.x : c.dummy) * Lat<D>::row_bytes + c.dofs[0];
  const uint32_t off1 = (uint32_t)(ok1 ? e.y : c.dummy) * Lat<D>::row_bytes + c.dofs[1];
#pragma unroll
  for (int k = 0; k < Lat<D>::lines; ++k) {
    dma16_sbase(off0, kvb + 128 * k, tile + 1024 * k);
    dma16_sbase(off1, kvb + 128 * k, tile + Lat<D>::group_bytes + 1024 * k);
  }
  return pd_valid(c, j);
}

// the sources of step j's copies and the validity bits of its 16 keys (key r <-> bit r)
struct PdSrc {
  const uint8_t* base;  // the latent (uniform)
  uint32_t off0;        // byte offset of this lane's 16 bytes of row er's first line
  uint32_t off1;        // ... of row 8 + er
  uint32_t vbits;
  int2 rows;            // the rows copied for keys er and 8 + er
};
template <int D>
__device__ __forceinline__ PdSrc pd_prep(const PdCtx& c, const uint8_t* kvb, int2 e, int j) {
  const bool ok0 = kPKeys * j + c.er < c.cols;
  const bool ok1 = kPKeys * j + 8 + c.er < c.cols;
  PdSrc p;
  p.base = kvb;
  p.rows = int2{ok0 ? e.x : c.dummy, ok1 ? e.y : c.dummy};
  p.off0 = (uint32_t)p.rows.x * Lat<D>::row_bytes + c.dofs[0];
  p.off1 = (uint32_t)p.rows.y * Lat<D>::row_bytes + c.dofs[1];
  p.vbits = pd_valid(c, j);
  return p;
}
// the two copies (row groups 0 and 1) of line k
template <int D>
__device__ __forceinline__ void pd_copy_line(const PdSrc& p, uint32_t tile, int k) {
  dma16_sbase(p.off0, p.base + 128 * k, tile + 1024 * k);
  dma16_sbase(p.off1, p.base + 128 * k, tile + Lat<D>::group_bytes + 1024 * k);
}

__device__ __forceinline__ int2 pd_entries(const PdCtx& c, int j) {
  const int i0 = min(kPKeys * j + c.er, c.cols - 1), i1 = min(kPKeys * j + 8 + c.er, c.cols - 1);
  int x0 = (int)pt_sorted[i0], x1 = (int)pt_sorted[i1];
  if (c.multi) {
    // the windows of the step's first and last entries (uniform); entries of a step that
    // crosses a window start count the starts below them one by one
    const int first = kPKeys * j, last = min(first + kPKeys - 1, c.cols - 1);
    const int wa = __popcll(ballot(c.lane >= 1 && c.wstart <= first));
    const int wb = __popcll(ballot(c.lane >= 1 && c.wstart <= last));
    int h0 = wa, h1 = wa;
    for (int w = wa + 1; w <= wb; ++w) {
      const int st = __builtin_amdgcn_readlane(c.wstart, w);
      h0 += i0 >= st ? 1 : 0;
      h1 += i1 >= st ? 1 : 0;
    }
    x0 |= h0 << 16;
    x1 |= h1 << 16;
  }
  return int2{x0, x1};
}

// S^T[key 4 g + jj][head n] (raw), one accumulation chain (dependent 16x16x32 MFMAs issue at
// full rate); K reads kPQAhead MFMAs ahead
template <int D>
__device__ __forceinline__ f32x4 pd_qk(const PdCtx& c, const uint8_t* tile, const bf16x8 (&qreg)[Lat<D>::loads]) {
  auto kread = [&](int s) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(tile + c.kofs[s & 1] + 1024 * (s >> 1));
  };
  bf16x8 kw[kPQAhead];
#pragma unroll
  for (int s = 0; s < kPQAhead; ++s) kw[s] = kread(s);
  f32x4 acc = {};
#pragma unroll
  for (int s = 0; s < Lat<D>::loads; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    acc = mfma16x16x32(kw[s % kPQAhead], qreg[s], acc);
    if (s + kPQAhead < Lat<D>::loads) kw[s % kPQAhead] = kread(s + kPQAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
  return acc;
}

// O^T += V^T P^T over the tile, which is refilled as it goes with the rows of a later step
// (`next`): the lines past the values (dims 512..575 of a 576-wide row, read only by S)
// first, then line k as soon as the MFMA of column block 4 k + 3 has consumed the last read
// of that line.  Spread over the MFMAs,
// the copies do not stall the wave on the CU's address path as a burst of 18 would.
template <int D>
__device__ __forceinline__ void pd_pv(const PdCtx& c, const uint8_t* tile, s16x4_t bop, f32x4 (&o)[kDv / 16],
                                      const PdSrc& next) {
  const uint32_t tl = lds_addr(tile);
  auto vread = [&](int cb) -> u16x4 { return lds_read_tr16(tile + c.rofs[cb & 3] + 1024 * (cb >> 2)); };
  u16x4 vw[kPVAhead];
#pragma unroll
  for (int i = 0; i < kPVAhead; ++i) vw[i] = vread(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = kDv / 64; k < Lat<D>::lines; ++k) pd_copy_line<D>(next, tl, k);
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) {
    __builtin_amdgcn_sched_barrier(0);
    o[cb] = mfma16x16x16(__builtin_bit_cast(s16x4_t, vw[cb % kPVAhead]), bop, o[cb]);
    if (cb + kPVAhead < kDv / 16) vw[cb % kPVAhead] = vread(cb + kPVAhead);
    if ((cb & 3) == 3) {
      // (after the MFMA: its wait for the operand read orders the copy behind the line's
      // last read)
      __builtin_amdgcn_sched_barrier(0);
      pd_copy_line<D>(next, tl, cb >> 2);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// invalid keys -> -inf (kScaled: valid scores times their row scales ks); returns the max of
// this lane's 4 scores
template <bool kScaled>
__device__ __forceinline__ float pd_mask(int g, const f32x4& sacc, uint32_t vbits, float (&sv)[4], f32x4 ks) {
  const uint32_t mine = vbits >> (4 * g);
  float mt = kNegInf;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)mine, jj, 1);  // all ones if valid
    // (a scalar copy: bit casts of vector elements misread)
    const float raw = kScaled ? sacc[jj] * ks[jj] : sacc[jj];
    sv[jj] = __builtin_bit_cast(float, (sel & __builtin_bit_cast(uint32_t, raw)) | (~sel & 0xff800000u));
    mt = fmaxf(mt, sv[jj]);
  }
  return mt;
}

template <bool kScaled>
__device__ __forceinline__ s16x4_t pd_probs(float sc, const float (&sv)[4], float m, float& l, f32x4 ks) {
  const float nm = m == kNegInf ? 0.f : -m;
  bf16x4 pb;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float p = fast_exp2(__builtin_fmaf(sv[jj], sc, nm));
    l += p;
    pb[jj] = (__bf16)(kScaled ? p * ks[jj] : p);
  }
  return __builtin_bit_cast(s16x4_t, pb);
}

template <int D, bool kScaled>
__global__ __launch_bounds__(64) void pertoken_sorted_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, int64_t ld, int T, int H, int S, int cols,
    int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ kscale, int per_row, const int32_t* __restrict__ skip) {
  if (skip != nullptr && uniform(*skip) != 0) return;  // (another routing was chosen on the device)
  const int nb = H >> 4;
  const int item = xcd_chunked_block((int)blockIdx.x, (int)gridDim.x, 16 * (H >> 4));  // (16 tokens)
  const int tq = item / nb;
  const int token = T - 1 - tq;
  const int hb = item - tq * nb;
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  int64_t pos64 = q_pos_offset + token;
  if (pos64 > S - 1) pos64 = S - 1;  // positions beyond S - 1 cannot be selected
  const int pos = uniform((int)pos64);

  // queries of head n, dims 32 s + 8 g .. + 8 (the B operand of S^T = K Q^T), negated for a
  // negative scale; completed before any asynchronous copy is in flight
  bf16x8 qreg[Lat<D>::loads];
  {
    const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
    const uint16_t* qrow = q + ((size_t)token * H + hb * 16 + n) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < Lat<D>::loads; ++s) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 32 * s);
      w ^= qsign;
      qreg[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  uint16_t* orow = out + ((size_t)token * H + hb * 16 + n) * kDv + 4 * g;
  float* lse_at = lse + (size_t)token * H + hb * 16 + n;
  int wstart;
  const int nsel = pt_sort(topk + (size_t)token * ld, cols, pos, lane, wstart);
#pragma unroll
  for (int s = 0; s < Lat<D>::loads; ++s) asm volatile("" : : "v"(qreg[s]));
  if (nsel == 0) {  // nothing selected: zero output, LSE -inf
    const f32x4 z[kDv / 16] = {};
    pt_write(g, z, 0.f, kNegInf, orow, lse_at);
    return;
  }
  if (nsel > kPSortMax) {  // more valid entries than the list holds: the register-ring walk
    pt_ring_token<D, kScaled>(q, kv, topk, ld, H, S, cols, q_pos_offset, scale_log2, out, lse, token, hb, kscale,
                              per_row);
    return;
  }
  const PdCtx c = pd_context<D>(pos, nsel, scale_log2, wstart);
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  uint8_t* const tile0 = pt_tile;
  uint8_t* const tile1 = reinterpret_cast<uint8_t*>(&pt_q[0][0]);

  // An even number of steps (an odd count gets one all-masked step, which adds nothing);
  // step j reads tile j % 2, and once its last operand read has been consumed the tile
  // receives step j + 2's rows, in flight during step j + 1.  Past the list the copies
  // fetch the token's own row and are masked.
  const int nsteps = (nsel + kPKeys - 1) / kPKeys;
  const int nsteps2 = nsteps + (nsteps & 1);
  float m_ref = kNegInf;  // head n's reference (log2 units); equal in the 4 lane groups
  float l_run = 0.f;      // this lane's partial sum (keys 4 g .. 4 g + 3 of every step)
  f32x4 o[kDv / 16];
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 sa = {1.f, 1.f, 1.f, 1.f}, sb = sa;  // kScaled: this lane's row scales of the tiles' steps
  const PdSrc s0 = pd_prep<D>(c, kvb, pd_entries(c, 0), 0);
  const PdSrc s1 = pd_prep<D>(c, kvb, pd_entries(c, 1), 1);
  if (kScaled) {
    sa = step_scales_mine(step_scales_load(kscale, per_row, s0.rows), g);
    sb = step_scales_mine(step_scales_load(kscale, per_row, s1.rows), g);
    // (consumed here, before any copy is in flight: the compiler may fetch these scales with
    // a vector load, and one it still took for pending at the loop would put vector-memory
    // waits, which also wait for the copies in flight, into every step)
    asm volatile("" : "+v"(sa), "+v"(sb));
  }
  uint32_t va = pd_issue<D>(c, kvb, pd_entries(c, 0), 0, lds_addr(tile0));
  uint32_t vb = pd_issue<D>(c, kvb, pd_entries(c, 1), 1, lds_addr(tile1));
  int2 e_next = pd_entries(c, 2);
  bool over = false;
  auto step = [&](int j, const uint8_t* tile, uint32_t& vbuf, f32x4& sbuf) {
    wait_vmcnt<2 * Lat<D>::lines>();  // step j's copies have landed (step j + 1's may be in flight)
    const f32x4 sacc = pd_qk<D>(c, tile, qreg);
    // the tile takes step j + 2's rows during its PV; kScaled: their scales are loaded under
    // this step's softmax and selected after its PV
    const PdSrc next = pd_prep<D>(c, kvb, e_next, j + 2);
    StepScales st;
    if (kScaled) st = step_scales_load(kscale, per_row, next.rows);
    float sv[4];
    const float mt = pd_mask<kScaled>(g, sacc, vbuf, sv, sbuf) * c.sc;
    // a head's first valid scores set its reference (its O and l are still zero)
    if (ballot(m_ref == kNegInf && mt != kNegInf) != 0) {
      const float mh = max_over_rowgroups(mt);
      m_ref = m_ref == kNegInf ? mh : m_ref;
    }
    over |= ballot(mt > m_ref + kPSlack) != 0;
    e_next = pd_entries(c, j + 3);
    pd_pv<D>(c, tile, pd_probs<kScaled>(c.sc, sv, m_ref, l_run, sbuf), o, next);
    vbuf = next.vbits;
    if (kScaled) sbuf = step_scales_mine(st, g);
  };
  for (int j = 0; j < nsteps2; j += 2) {
    step(j, tile0, va, sa);
    step(j + 1, tile1, vb, sb);
  }
  wait_vmcnt<0>();  // the copies issued past the list
  if (over) {
    // the exact routine reads the queries from the second tile's area
#pragma unroll
    for (int s = 0; s < Lat<D>::loads; ++s) pt_q[s][lane] = __builtin_bit_cast(uint4, qreg[s]);
    __syncthreads();
    pt_exact<D, true, kScaled>(kv, topk, ld, S, nsel, q_pos_offset, scale_log2, token, orow, lse_at, wstart,
                               kscale, per_row, c.dummy);
    return;
  }
  pt_write(g, o, l_run, m_ref, orow, lse_at);
}

template <int D, bool kScaled>
static void launch_pertoken(const uint16_t* q, const uint16_t* kv, const int32_t* topk, int64_t ld, int T,
                            int H, int S, int cols, int64_t q_pos_offset, float scale, uint16_t* out,
                            float* lse, hipStream_t stream, const float* kscale, int per_row,
                            const int32_t* skip) {
  const long long items = (long long)T * (H / 16);
  if (S <= kPSortRows)
    hipLaunchKernelGGL((pertoken_sorted_kernel<D, kScaled>), dim3((unsigned)items), dim3(64), 0, stream, q, kv,
                       topk, ld, T, H, S, cols, q_pos_offset, scale * kLog2e, out, lse, kscale, per_row, skip);
  else
    hipLaunchKernelGGL((pertoken_attn_kernel<D, kScaled>), dim3((unsigned)items), dim3(64), 0, stream, q, kv,
                       topk, ld, T, H, S, cols, q_pos_offset, scale * kLog2e, out, lse, kscale, per_row, skip);
}

hipError_t launch_pertoken_attn(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                float scale, uint16_t* out, float* lse, hipStream_t stream, int d_qk,
                                const float* kscale, int per_row, const int32_t* skip) {
  if ((long long)T * (H / 16) == 0) return hipSuccess;
  if (d_qk == 512) {
    if (kscale)
      launch_pertoken<512, true>(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse, stream, kscale,
                                 per_row, skip);
    else
      launch_pertoken<512, false>(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse, stream, kscale,
                                  per_row, skip);
  } else {
    if (kscale)
      launch_pertoken<576, true>(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse, stream, kscale,
                                 per_row, skip);
    else
      launch_pertoken<576, false>(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse, stream, kscale,
                                  per_row, skip);
  }
  return hipGetLastError();
}

}  // namespace dsa
