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
// MI355X design: one wave per (token, 16-head block), one wave per workgroup
// (no barriers), one wave per SIMD:
//  * the token's top-k row is consumed 16 entries at a time; lane (g, n) owns
//    entry n of a step and loads 16-byte chunks 4 s + g (s = 0..17) of that
//    latent row straight into registers.  Two register buffers form a ring: a
//    step's buffer is refilled with the rows two steps ahead as soon as its
//    QK MFMAs have read it, so up to two steps (36 KiB) are in flight per
//    wave -- a gather of scattered 1152-byte rows is latency bound, and LDS
//    capacity no longer limits the bytes in flight.  Invalid entries (-1, past
//    the row, beyond the token's position) load the token's own row and are
//    masked;
//  * S^T = K Q^T takes the rows from registers as the A operand of
//    v_mfma_f32_16x16x32_bf16, in three independent accumulation chains; the
//    B operand (the 16 heads' queries) is re-read every step from a
//    lane-private LDS area, since the register file holds the ring;
//  * the value part of the rows goes through a 16 KiB LDS tile (XOR-swizzled,
//    free of bank conflicts for both the 16-byte writes and the transposed
//    reads) so that ds_read_b64_tr_b16 can hand V^T to O^T = V^T P^T
//    (v_mfma_f32_16x16x16_bf16); the probabilities leave the accumulators
//    directly as the B operand;
//  * fp32 softmax in base 2 on raw scores (the scale is folded into the
//    exponent's FMA; a negative scale negates the queries) against a per-head
//    reference fixed at the head's first valid scores, so O is only ever
//    written by MFMAs and stays in the accumulation registers; each lane keeps
//    its own partial sum, so the common path has no cross-lane reduction.
//    Probabilities may exceed 1 by up to 2^64 (safe for bf16 P and fp32 O and
//    l); a token with a score beyond that is recomputed by an exact two-pass
//    routine (max first), which is not met with ordinary inputs;
//  * token order is reversed (long causal rows first) and block ids are
//    remapped so each XCD runs a contiguous token range: neighbouring tokens,
//    which share most of their rows, then hit the same L2.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kPKeys = 16;                  // keys per step
constexpr int kPLoads = kDqk / 32;          // 16-byte chunks per lane per step (18)
constexpr int kPVLoads = kDv / 32;          // of which hold value dims (16)
constexpr int kPRowBytes = kDqk * 2;        // 1152
constexpr int kPVRowBytes = kDv * 2;        // 1024: one V row in the LDS tile
constexpr float kPSlack = 64.f;             // log2 of the largest probability allowed

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(s16x4_t a, s16x4_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// LDS of the (single-wave) workgroup: the V tile of the current step -- chunk c (16 B,
// 0..63) of row r (0..15) at r * 1024 + 16 (c ^ vswz(r)) -- and the queries, lane-private:
// lane l's chunk s at pt_q[s][l].
__shared__ __align__(16) uint8_t pt_vtile[kPKeys * kPVRowBytes];
__shared__ __align__(16) uint4 pt_q[kPLoads][64];

__device__ __forceinline__ int vswz(int r) { return (2 * r + (r >> 3)) & 15; }

// What one wave needs to walk its token's row.
struct PtCtx {
  const int32_t* trow;  // the token's top-k row
  const uint8_t* kvb;   // latent base + 16 g (this lane's chunk column)
  int cols, pos, lane, g, n;
  float sc;             // |scale| * log2(e)
  int wofs[4];          // LDS V-tile store offsets (per chunk group s % 4)
  int rofs[8];          // LDS V-tile transposed-read offsets (per column block cb % 8)
};

// this lane's entry of step j (column 16 j + n, clamped into the row)
__device__ __forceinline__ int32_t pt_entry(const PtCtx& c, int j) {
  return c.trow[min(kPKeys * j + c.n, c.cols - 1)];
}

// start the loads of step j's rows into `buf`; returns the validity bits (key r <-> bit r)
__device__ __forceinline__ uint32_t pt_issue(const PtCtx& c, int32_t e, int j, uint4 (&buf)[kPLoads]) {
  const bool ok = kPKeys * j + c.n < c.cols && e >= 0 && e <= c.pos;
  const uint4* src = reinterpret_cast<const uint4*>(c.kvb + (size_t)(ok ? e : c.pos) * kPRowBytes);
#pragma unroll
  for (int s = 0; s < kPLoads; ++s) buf[s] = src[4 * s];
  return (uint32_t)ballot(ok) & 0xffffu;
}

__device__ __forceinline__ void pt_store_v(const PtCtx& c, const uint4 (&buf)[kPLoads]) {
#pragma unroll
  for (int s = 0; s < kPVLoads; ++s)
    *reinterpret_cast<uint4*>(pt_vtile + c.wofs[s & 3] + 256 * (s >> 2)) = buf[s];
}

// S^T[key 4 g + jj][head n] (raw) of the rows in `buf`, in three independent chains
__device__ __forceinline__ f32x4 pt_qk(const PtCtx& c, const uint4 (&buf)[kPLoads]) {
  // (the query address is made opaque: hoisted out of a loop, the 18 reads would pin 72
  // registers for the whole token)
  const uint8_t* qb = reinterpret_cast<const uint8_t*>(&pt_q[0][0]) + loop_local(16 * c.lane);
  f32x4 acc[3] = {};
#pragma unroll
  for (int s = 0; s < kPLoads; ++s)
    acc[s % 3] = mfma16x16x32(__builtin_bit_cast(bf16x8, buf[s]),
                              *reinterpret_cast<const bf16x8*>(qb + 1024 * s), acc[s % 3]);
  return acc[0] + acc[1] + acc[2];
}

// invalid keys -> -inf; returns the max of this lane's 4 scores
__device__ __forceinline__ float pt_mask(const PtCtx& c, const f32x4& sacc, uint32_t vbits, float (&sv)[4]) {
  const uint32_t mine = vbits >> (4 * c.g);
  float mt = kNegInf;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)mine, jj, 1);  // all ones if valid
    const float raw = sacc[jj];  // (a scalar copy: bit casts of vector elements misread)
    sv[jj] = __builtin_bit_cast(float, (sel & __builtin_bit_cast(uint32_t, raw)) | (~sel & 0xff800000u));
    mt = fmaxf(mt, sv[jj]);
  }
  return mt;
}

// P = 2^(s sc - m) (bf16, as the B operand P^T[key 4 g + jj][head n]); adds to l
__device__ __forceinline__ s16x4_t pt_probs(const PtCtx& c, const float (&sv)[4], float m, float& l) {
  const float nm = m == kNegInf ? 0.f : -m;
  bf16x4 pb;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float p = fast_exp2(__builtin_fmaf(sv[jj], c.sc, nm));
    l += p;
    pb[jj] = (__bf16)p;
  }
  return __builtin_bit_cast(s16x4_t, pb);
}

// O^T[col 16 cb + 4 g + jj][head n] += V^T P^T
__device__ __forceinline__ void pt_pv(const PtCtx& c, s16x4_t bop, f32x4 (&o)[kDv / 16]) {
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) {
    const u16x4 a = lds_read_tr16(pt_vtile + c.rofs[cb & 7] + 256 * (cb >> 3));
    o[cb] = mfma16x16x16(__builtin_bit_cast(s16x4_t, a), bop, o[cb]);
  }
}

__device__ __forceinline__ void pt_write(const PtCtx& c, const f32x4 (&o)[kDv / 16], float l_part, float m,
                                         uint16_t* orow, float* lse_at) {
  const float l = sum_over_rowgroups(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) {
    const bf16x4 w = {(__bf16)(o[cb][0] * inv), (__bf16)(o[cb][1] * inv), (__bf16)(o[cb][2] * inv),
                      (__bf16)(o[cb][3] * inv)};
    *reinterpret_cast<bf16x4*>(orow + 16 * cb) = w;
  }
  if (c.g == 0) *lse_at = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
}

// Exact two-pass routine: head n's max over the whole row first, then the softmax
// against it (no probability exceeds 1).  Both passes share pt_qk / pt_mask with the main
// loop, so their scores are bit-identical.
__device__ __noinline__ void pt_exact(const PtCtx& c, uint16_t* orow, float* lse_at) {
  const int nsteps = (c.cols + kPKeys - 1) / kPKeys;
  float m = kNegInf;
  for (int j = 0; j < nsteps; ++j) {
    uint4 buf[kPLoads];
    const uint32_t vbits = pt_issue(c, pt_entry(c, j), j, buf);
    float sv[4];
    m = fmaxf(m, pt_mask(c, pt_qk(c, buf), vbits, sv));
  }
  m = max_over_rowgroups(m) * c.sc;
  float l = 0.f;
  f32x4 o[kDv / 16];
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nsteps; ++j) {
    uint4 buf[kPLoads];
    const uint32_t vbits = pt_issue(c, pt_entry(c, j), j, buf);
    pt_store_v(c, buf);
    float sv[4];
    pt_mask(c, pt_qk(c, buf), vbits, sv);
    pt_pv(c, pt_probs(c, sv, m, l), o);
  }
  pt_write(c, o, l, m, orow, lse_at);
}

__global__ __launch_bounds__(64) void pertoken_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ topk, int64_t ld, int T, int H, int S, int cols,
    int64_t q_pos_offset, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int nb = H >> 4;
  const int item = xcd_logical_block((int)blockIdx.x, (int)gridDim.x);
  const int tq = item / nb;
  const int token = T - 1 - tq;
  const int hb = item - tq * nb;

  PtCtx c;
  c.lane = threadIdx.x;
  c.g = c.lane >> 4;
  c.n = c.lane & 15;
  int64_t pos64 = q_pos_offset + token;
  if (pos64 > S - 1) pos64 = S - 1;  // positions beyond S - 1 cannot be selected
  c.pos = uniform((int)pos64);
  c.cols = cols;
  c.trow = topk + (size_t)token * ld;
  c.kvb = reinterpret_cast<const uint8_t*>(kv) + 16 * c.g;
  c.sc = fabsf(scale_log2);
  // LDS V tile.  Stores: lane (g, n) writes chunk 4 s + g of row n.  Transposed reads for
  // O^T block cb (cols 16 cb .. + 15): lane (g, i) of a 16-lane group addresses row
  // 4 g + i / 4, cols 16 cb + 4 (i % 4) .. + 3 (chunk 2 cb + (i % 4) / 2, half i % 2), so
  // that output lane (g, n) receives V[key 4 g + jj][col 16 cb + n], jj = 0..3.
  {
    const int wx = c.g ^ vswz(c.n);
    const int rr = 4 * c.g + (c.n >> 2);
    const int rx = ((c.n >> 1) & 1) ^ vswz(rr);
#pragma unroll
    for (int u = 0; u < 4; ++u) c.wofs[u] = c.n * kPVRowBytes + 16 * (wx ^ (4 * u));
#pragma unroll
    for (int b = 0; b < 8; ++b) c.rofs[b] = rr * kPVRowBytes + 8 * (c.n & 1) + 16 * (rx ^ (2 * b));
  }

  // queries of head n, dims 32 s + 8 g .. + 8 (the B operand of S^T = K Q^T); a negative
  // scale is applied as |scale| on negated queries so the max can be taken on raw scores
  {
    const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
    const uint16_t* qrow = q + ((size_t)token * H + hb * 16 + c.n) * kDqk + 8 * c.g;
#pragma unroll
    for (int s = 0; s < kPLoads; ++s) {
      uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * s);
      w.x ^= qsign; w.y ^= qsign; w.z ^= qsign; w.w ^= qsign;
      pt_q[s][c.lane] = w;
    }
  }
  uint16_t* orow = out + ((size_t)token * H + hb * 16 + c.n) * kDv + 4 * c.g;
  float* lse_at = lse + (size_t)token * H + hb * 16 + c.n;
  if (cols == 0) {  // nothing selected: zero output, LSE -inf
    const f32x4 z[kDv / 16] = {};
    pt_write(c, z, 0.f, kNegInf, orow, lse_at);
    return;
  }

  // The main loop runs an even number of steps (an odd count gets one all-masked step,
  // which adds nothing), so that it has a single exit.  Step j lives in register buffer
  // j % 2; its QK MFMAs and V stores consume the buffer, which then receives step j + 2's
  // rows, in flight during step j's softmax and PV and all of step j + 1.  The entry of
  // step j + 3 is read before step j + 2's loads, so that waiting for an entry never
  // waits for rows issued after it.
  const int nsteps = (cols + kPKeys - 1) / kPKeys;
  const int nsteps2 = nsteps + (nsteps & 1);
  float m_ref = kNegInf;  // head n's reference (log2 units); equal in the 4 lane groups
  float l_run = 0.f;      // this lane's partial sum (keys 4 g .. 4 g + 3 of every step)
  f32x4 o[kDv / 16];
#pragma unroll
  for (int cb = 0; cb < kDv / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ra[kPLoads], rb[kPLoads];
  uint32_t va = 0, vb = 0;
  int32_t e_next = 0;  // entry of the step whose loads start next
  {  // issue order as in the loop (entry, rows, entry, rows), pinned by scheduling
     // barriers: the wait counts at the loop head merge this order with the loop's
    const int32_t e0 = pt_entry(c, 0);
    const int32_t e1 = pt_entry(c, 1);
    __builtin_amdgcn_sched_barrier(0);
    va = pt_issue(c, e0, 0, ra);
    __builtin_amdgcn_sched_barrier(0);
    e_next = pt_entry(c, 2);
    __builtin_amdgcn_sched_barrier(0);
    vb = pt_issue(c, e1, 1, rb);
    __builtin_amdgcn_sched_barrier(0);
  }
  // one step; `over` becomes true when a score exceeds the reference by more than the
  // slack (the loop still runs to its end, and its result is then discarded)
  bool over = false;
  auto step = [&](int j, uint4 (&buf)[kPLoads], uint32_t& vbuf) {
    pt_store_v(c, buf);
    const f32x4 sacc = pt_qk(c, buf);
    const uint32_t vbits = vbuf;
    // the refill must not be scheduled above the reads of the buffer it overwrites
    __builtin_amdgcn_sched_barrier(0);
    {  // (unconditional: past the row the loads are masked dummies, and the wait
       // counts stay exact only on a branch-free path)
      const int32_t e = e_next;
      e_next = pt_entry(c, j + 3);
      __builtin_amdgcn_sched_barrier(0);
      vbuf = pt_issue(c, e, j + 2, buf);
    }
    __builtin_amdgcn_sched_barrier(0);
    float sv[4];
    const float mt = pt_mask(c, sacc, vbits, sv) * c.sc;
    // a head's first valid scores set its reference (its O and l are still zero)
    if (ballot(m_ref == kNegInf && mt != kNegInf) != 0) {
      const float mh = max_over_rowgroups(mt);
      m_ref = m_ref == kNegInf ? mh : m_ref;
    }
    over |= ballot(mt > m_ref + kPSlack) != 0;
    pt_pv(c, pt_probs(c, sv, m_ref, l_run), o);
  };
  for (int j = 0; j < nsteps2; j += 2) {
    step(j, ra, va);
    step(j + 1, rb, vb);
  }
  if (over) {
    pt_exact(c, orow, lse_at);
    return;
  }
  pt_write(c, o, l_run, m_ref, orow, lse_at);
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
