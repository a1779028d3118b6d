// C-ABI host layer of libdsa_prefill.so: argument checks, then kernel launches
// on the caller's stream.  Nothing here allocates, frees or synchronizes.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "dsa_prefill.h"
#include "kernels.h"

namespace {

inline bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

// the kernels fold the scale into exponent FMAs on raw scores: it must be finite and nonzero
inline bool scale_ok(float s) { return s == s && s != 0.f && s - s == 0.f; }

// latent widths: 576 (512 + 64 rope dims) or 512 (no rope part); values are the first 512
// dims of a row either way
constexpr int kValueDim = 512;
inline bool latent_ok(int d_qk, int d_v) { return (d_qk == 576 || d_qk == 512) && d_v == kValueDim; }

// MHA geometries (qk_nope, qk_rope, v) of the masked and dense forms
inline bool mha_nope(int dn, int dr, int dv) { return dn == 256 && dr == 0 && dv == 256; }
inline bool mha_rope(int dn, int dr, int dv) {
  return (dn == 192 && dr == 64 && dv == 256) || (dn == 128 && dr == 64 && dv == 128);
}

// host checks of a batch description (its device contents are never errors)
inline bool batch_shape_ok(int T, int cols, int64_t ld, int R, int64_t bt_ld, int page_size, int num_slots) {
  return T >= 0 && cols >= 0 && ld >= cols && R >= 1 && bt_ld >= 1 && page_size >= 1 && num_slots >= 1;
}
inline bool batch_ptrs_ok(const int32_t* cu, const int32_t* kv_lens, const int32_t* q_pos_start,
                          const int32_t* block_table) {
  return cu && kv_lens && q_pos_start && block_table;
}
inline bool batch_aligned(const int32_t* cu, const int32_t* kv_lens, const int32_t* q_pos_start,
                          const int32_t* block_table) {
  return aligned_to(cu, 4) && aligned_to(kv_lens, 4) && aligned_to(q_pos_start, 4) && aligned_to(block_table, 4);
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size or leading dimension is out of range";
    case DSA_ERR_UNSUPPORTED: return "unsupported head count, head dimensions or scale";
    case DSA_ERR_ALIGN: return "a pointer is not aligned as required";
    case DSA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case DSA_ERR_CAPACITY: return "the work needs more than the library's static scratch (DSA_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int dsa_union_pad(int G, int cols) {
  if (G < 1 || G > 8 || cols < 0) return DSA_ERR_SHAPE;
  const long long v = ((long long)G * cols + 63) / 64 * 64;
  if (v > INT_MAX) return DSA_ERR_SHAPE;
  return (int)v;
}

// Routing choice for one chunk ("[2/N][Attention] Enable masked MHA for sparse MLA prefills",
// Purpose section and its heuristic commit: below some length the masked MHA beats the sparse
// MQA kernels, and a chunk no longer than the top-k needs no mask at all).  The thresholds
// are MI355X measurements of this library's kernels: chunks of L tokens from position 0 with
// top-2048 (8-token locality), the MQA forms over the 576- and the 512-wide latent (c lies
// between the two widths' crossovers, nearer the 576-wide one).  Masked and sparse times
// cross where the mean number of causal keys per query token reaches c * k (masked time grows
// with the causal pairs, sparse time with the selected ones).
namespace {
double masked_threshold(int H, int mha_dv, bool grouped) {
  // {H 16, 32, 64 against grouped; 128 against per-token (G = 1); other H against per-token}
  static const double kQk256[5] = {2.4, 1.95, 1.7, 1.4, 3.4};  // (256, 0, 256), (192, 64, 256)
  static const double kDsv[5] = {3.6, 3.05, 2.75, 2.4, 5.5};     // (128, 64, 128)
  const double* c = mha_dv == 128 ? kDsv : kQk256;
  if (!grouped) return H == 128 ? c[3] : c[4];
  return H == 16 ? c[0] : (H == 32 ? c[1] : c[2]);
}
}  // namespace

int dsa_select_routing(int T, int S, int64_t q_pos_offset, int H, int k, int mha_dv) {
  if (T < 0 || S < 1 || q_pos_offset < 0 || H < 1 || k < 1) return DSA_ERR_SHAPE;
  if (mha_dv != 0 && mha_dv != 256 && mha_dv != 128) return DSA_ERR_UNSUPPORTED;
  const bool mha = mha_dv != 0;
  const bool mqa_ok = H % 16 == 0 && H <= 128;
  const bool grouped_ok = mqa_ok && 128 % H == 0 && H < 128;
  if (!mqa_ok && !mha) return DSA_ERR_UNSUPPORTED;
  if (mha && q_pos_offset + (int64_t)T <= k) return DSA_ROUTING_DENSE;
  if (mha) {
    if (!mqa_ok) return DSA_ROUTING_MASKED;
    // mean over the chunk of min(S, p_t + 1), p_t = q_pos_offset + t
    const double first = (double)q_pos_offset + 1.0;
    double sum;
    if (first >= (double)S) {
      sum = (double)T * S;
    } else {
      const double n = fmin((double)T, (double)S - first + 1.0);  // tokens below the cap
      sum = n * first + n * (n - 1.0) / 2.0 + ((double)T - n) * S;
    }
    const double mean = T > 0 ? sum / T : 0.0;
    if (mean <= masked_threshold(H, mha_dv, grouped_ok) * k) return DSA_ROUTING_MASKED;
  }
  return grouped_ok ? DSA_ROUTING_GROUPED : DSA_ROUTING_PERTOKEN;
}

size_t dsa_masked_mha_workspace_bytes(int T, int S) {
  if (T < 0 || S < 0) return 0;
  return (size_t)T * (size_t)((S + 31) / 32) * sizeof(uint32_t);
}

int dsa_build_group_union(const int32_t* topk, int64_t ld, int T, int cols, int S,
                          int64_t q_pos_offset, int G, int union_pad, int32_t* union_idx,
                          int32_t* union_len, uint8_t* head_group_mask, void* stream) {
  if (T < 0 || cols < 0 || S < 1 || ld < cols || q_pos_offset < 0) return DSA_ERR_SHAPE;
  if (G < 1 || G > 8) return DSA_ERR_SHAPE;
  if (union_pad < 0 || union_pad % 64 != 0 || (long long)union_pad < (long long)G * cols)
    return DSA_ERR_SHAPE;
  if (T == 0) return DSA_OK;
  if ((cols > 0 && !topk) || !union_idx || !union_len || !head_group_mask) return DSA_ERR_NULL;
  if (!aligned_to(topk, 4) || !aligned_to(union_idx, 4) || !aligned_to(union_len, 4))
    return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_build_union(topk, ld, T, cols, S, q_pos_offset, G, union_pad,
                                               union_idx, union_len, head_group_mask,
                                               (hipStream_t)stream));
}

// Host checks of the grouped and per-token calls: DSA_OK when the call has work to enqueue,
// kNothingToDo for an empty one, else the (negative) status.
constexpr int kNothingToDo = 1;

static int grouped_check(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                         const int32_t* union_len, const uint8_t* head_group_mask, int T, int H, int S,
                         int union_pad, int d_qk, int d_v, float scale, const uint16_t* out,
                         const float* lse) {
  if (H != 16 && H != 32 && H != 64 && H != 128) return DSA_ERR_UNSUPPORTED;
  if (!latent_ok(d_qk, d_v) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (T < 0 || S < 1 || union_pad < 0 || union_pad % 32 != 0) return DSA_ERR_SHAPE;
  if (T == 0) return kNothingToDo;
  if (!q || !kv || !union_idx || !union_len || !head_group_mask || !out || !lse)
    return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(kv, 16) || !aligned_to(out, 16) || !aligned_to(lse, 4) ||
      !aligned_to(union_idx, 4) || !aligned_to(union_len, 4) || !aligned_to(head_group_mask, 4))
    return DSA_ERR_ALIGN;
  return DSA_OK;
}

static int pertoken_check(const uint16_t* q, const uint16_t* kv, const int32_t* topk, int64_t ld, int T,
                          int H, int S, int cols, int64_t q_pos_offset, int d_qk, int d_v, float scale,
                          const uint16_t* out, const float* lse) {
  if (H < 16 || H > 128 || H % 16 != 0) return DSA_ERR_UNSUPPORTED;
  if (!latent_ok(d_qk, d_v) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (T < 0 || S < 1 || cols < 0 || ld < cols || q_pos_offset < 0) return DSA_ERR_SHAPE;
  if (T == 0) return kNothingToDo;
  if (!q || !kv || (cols > 0 && !topk) || !out || !lse) return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(kv, 16) || !aligned_to(out, 16) || !aligned_to(lse, 4) ||
      !aligned_to(topk, 4))
    return DSA_ERR_ALIGN;
  return DSA_OK;
}

static hipError_t pertoken_launch(const uint16_t* q, const uint16_t* kv, const int32_t* topk, int64_t ld,
                                  int T, int H, int S, int cols, int64_t q_pos_offset, int d_qk, float scale,
                                  uint16_t* out, float* lse, hipStream_t stream, const float* kscale = nullptr,
                                  int scale_per_row = 0) {
  if (H == 128)
    return dsa::launch_pertoken_rows128(q, kv, topk, ld, T, S, cols, q_pos_offset, scale, out, lse, stream,
                                        d_qk, kscale, scale_per_row);
  return dsa::launch_pertoken_attn(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse, stream,
                                   d_qk, kscale, scale_per_row);
}

// the FP8 latent arguments (kv8 [S, d_qk] codes, kv_scale, the bf16 workspace)
static int fp8_check(const uint8_t* kv8, const float* kv_scale, int scale_per_row, const uint16_t* kv_ws) {
  if (scale_per_row != 0 && scale_per_row != 1) return DSA_ERR_SHAPE;
  if (!kv8 || !kv_scale || !kv_ws) return DSA_ERR_NULL;
  if (!aligned_to(kv8, 16) || !aligned_to(kv_scale, 4) || !aligned_to(kv_ws, 16)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

int dsa_sparse_prefill_grouped(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                               const int32_t* union_len, const uint8_t* head_group_mask, int T,
                               int H, int S, int union_pad, int d_qk, int d_v, float scale,
                               uint16_t* out, float* lse, void* stream) {
  const int st = grouped_check(q, kv, union_idx, union_len, head_group_mask, T, H, S, union_pad, d_qk, d_v,
                               scale, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  return launch_status(dsa::launch_grouped_attn(q, kv, union_idx, union_len, head_group_mask, T,
                                                H, S, union_pad, scale, out, lse,
                                                (hipStream_t)stream, nullptr, 0, d_qk));
}

int dsa_sparse_prefill_pertoken(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                int d_qk, int d_v, float scale, uint16_t* out, float* lse,
                                void* stream) {
  const int st = pertoken_check(q, kv, topk, ld, T, H, S, cols, q_pos_offset, d_qk, d_v, scale, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  return launch_status(pertoken_launch(q, kv, topk, ld, T, H, S, cols, q_pos_offset, d_qk, scale, out, lse,
                                       (hipStream_t)stream));
}

// per-token cost of the grouped form's 128-row tiles, per 32 selections (measured on MI355X
// with this library's kernels, 576-wide latent, 16k-token chunks, locality and uniform top-k)
static double route_rho(int H) { return H == 16 ? 0.22 : (H == 32 ? 0.46 : 0.94); }

// sum over the chunk of min(cols, S, p_t + 1), p_t = q_pos_offset + t: the selections a
// token can make (an upper bound when rows hold -1 or out-of-range entries)
static double selections_bound(int T, int S, int64_t q_pos_offset, int cols) {
  const double c = (double)(cols < S ? cols : S);
  const double p1 = (double)q_pos_offset + 1.0;                  // p_0 + 1
  const double n1 = fmin((double)T, fmax(0.0, c - p1));           // tokens below the cap
  return n1 * p1 + n1 * (n1 - 1.0) / 2.0 + ((double)T - n1) * c;
}

int dsa_sparse_prefill_auto(const uint16_t* q, const uint16_t* kv, const int32_t* topk, int64_t ld, int T,
                            int H, int S, int cols, int64_t q_pos_offset, int d_qk, int d_v, float scale,
                            int union_pad, int32_t* union_idx, int32_t* union_len, uint8_t* head_group_mask,
                            int32_t* route, uint16_t* out, float* lse, void* stream) {
  if (H != 16 && H != 32 && H != 64) return DSA_ERR_UNSUPPORTED;
  const int G = 128 / H;
  int st = pertoken_check(q, kv, topk, ld, T, H, S, cols, q_pos_offset, d_qk, d_v, scale, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  st = grouped_check(q, kv, union_idx, union_len, head_group_mask, T, H, S, union_pad, d_qk, d_v, scale, out,
                     lse);
  if (st != DSA_OK) return st;
  if (union_pad % 64 != 0 || (long long)union_pad < (long long)G * cols) return DSA_ERR_SHAPE;
  if (!route) return DSA_ERR_NULL;
  if (!aligned_to(route, 4)) return DSA_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  const int NG = (T + G - 1) / G;
  const double limit = route_rho(H) * selections_bound(T, S, q_pos_offset, cols) / 32.0;
  hipError_t e = dsa::launch_build_union(topk, ld, T, cols, S, q_pos_offset, G, union_pad, union_idx, union_len,
                                         head_group_mask, s);
  if (e == hipSuccess) e = dsa::launch_route_by_union(union_len, NG, union_pad, limit, route, s);
  if (e == hipSuccess)
    e = dsa::launch_grouped_attn(q, kv, union_idx, union_len, head_group_mask, T, H, S, union_pad, scale, out,
                                 lse, s, nullptr, 0, d_qk, nullptr, 0, route);
  if (e == hipSuccess)
    e = dsa::launch_pertoken_attn(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse, s, d_qk, nullptr,
                                  0, route + 1);
  return launch_status(e);
}

int dsa_decode_latent_fp8(const uint8_t* kv8, int S, int d, uint16_t* out, void* stream) {
  if (d != 576 && d != 512) return DSA_ERR_UNSUPPORTED;
  if (S < 0) return DSA_ERR_SHAPE;
  if (S == 0) return DSA_OK;
  if (!kv8 || !out) return DSA_ERR_NULL;
  if (!aligned_to(kv8, 16) || !aligned_to(out, 16)) return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_decode_fp8(kv8, S, d, out, (hipStream_t)stream));
}

int dsa_sparse_prefill_grouped_fp8(const uint16_t* q, const uint8_t* kv8, const float* kv_scale,
                                   int scale_per_row, const int32_t* union_idx, const int32_t* union_len,
                                   const uint8_t* head_group_mask, int T, int H, int S, int union_pad,
                                   int d_qk, int d_v, float scale, uint16_t* kv_ws, uint16_t* out, float* lse,
                                   void* stream) {
  // (the bf16 checks see the workspace as the latent)
  int st = grouped_check(q, kv_ws, union_idx, union_len, head_group_mask, T, H, S, union_pad, d_qk, d_v,
                         scale, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  if ((st = fp8_check(kv8, kv_scale, scale_per_row, kv_ws)) != DSA_OK) return st;
  const hipError_t e = dsa::launch_decode_fp8(kv8, S, d_qk, kv_ws, (hipStream_t)stream);
  if (e != hipSuccess) return DSA_ERR_LAUNCH;
  return launch_status(dsa::launch_grouped_attn(q, kv_ws, union_idx, union_len, head_group_mask, T, H, S,
                                                union_pad, scale, out, lse, (hipStream_t)stream, nullptr, 0,
                                                d_qk, kv_scale, scale_per_row));
}

int dsa_sparse_prefill_pertoken_fp8(const uint16_t* q, const uint8_t* kv8, const float* kv_scale,
                                    int scale_per_row, const int32_t* topk, int64_t ld, int T, int H, int S,
                                    int cols, int64_t q_pos_offset, int d_qk, int d_v, float scale,
                                    uint16_t* kv_ws, uint16_t* out, float* lse, void* stream) {
  int st = pertoken_check(q, kv_ws, topk, ld, T, H, S, cols, q_pos_offset, d_qk, d_v, scale, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  if ((st = fp8_check(kv8, kv_scale, scale_per_row, kv_ws)) != DSA_OK) return st;
  const hipError_t e = dsa::launch_decode_fp8(kv8, S, d_qk, kv_ws, (hipStream_t)stream);
  if (e != hipSuccess) return DSA_ERR_LAUNCH;
  return launch_status(pertoken_launch(q, kv_ws, topk, ld, T, H, S, cols, q_pos_offset, d_qk, scale, out, lse,
                                       (hipStream_t)stream, kv_scale, scale_per_row));
}

int dsa_varlen_group_bound(int T, int R, int G) {
  if (T < 0 || R < 1 || G < 1 || G > 8) return DSA_ERR_SHAPE;
  const long long v = ((long long)T + G - 1) / G + R;
  return (int)(v < T ? v : T);
}

int dsa_convert_req_index_to_global(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                    const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                    const int32_t* q_pos_start, const int32_t* block_table, int64_t bt_ld,
                                    int page_size, int num_slots, int32_t* topk_global, void* stream) {
  if (!batch_shape_ok(T, cols, ld, R, bt_ld, page_size, num_slots)) return DSA_ERR_SHAPE;
  if (T == 0 || cols == 0) return DSA_OK;
  if (!topk || !topk_global || !batch_ptrs_ok(cu_seqlens_q, kv_lens, q_pos_start, block_table))
    return DSA_ERR_NULL;
  if (!aligned_to(topk, 4) || !aligned_to(topk_global, 4) ||
      !batch_aligned(cu_seqlens_q, kv_lens, q_pos_start, block_table))
    return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_convert_req_index(topk, ld, T, cols, R, cu_seqlens_q, kv_lens,
                                                     q_pos_start, block_table, bt_ld, page_size,
                                                     num_slots, topk_global, (hipStream_t)stream));
}

int dsa_build_group_union_varlen(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                 const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                 const int32_t* q_pos_start, const int32_t* block_table, int64_t bt_ld,
                                 int page_size, int num_slots, int G, int max_groups, int union_pad,
                                 int32_t* group_info, int32_t* union_idx, int32_t* union_len,
                                 uint8_t* head_group_mask, void* stream) {
  if (!batch_shape_ok(T, cols, ld, R, bt_ld, page_size, num_slots)) return DSA_ERR_SHAPE;
  if (G < 1 || G > 8 || max_groups < 0) return DSA_ERR_SHAPE;
  if (union_pad < 0 || union_pad % 64 != 0 || (long long)union_pad < (long long)G * cols)
    return DSA_ERR_SHAPE;
  if (max_groups == 0) return DSA_OK;
  if ((T > 0 && cols > 0 && !topk) || !group_info || !union_idx || !union_len || !head_group_mask ||
      !batch_ptrs_ok(cu_seqlens_q, kv_lens, q_pos_start, block_table))
    return DSA_ERR_NULL;
  if (!aligned_to(topk, 4) || !aligned_to(group_info, 8) || !aligned_to(union_idx, 4) ||
      !aligned_to(union_len, 4) || !batch_aligned(cu_seqlens_q, kv_lens, q_pos_start, block_table))
    return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_build_union_varlen(
      topk, ld, T, cols, R, cu_seqlens_q, kv_lens, q_pos_start, block_table, bt_ld, page_size, num_slots,
      G, max_groups, union_pad, group_info, union_idx, union_len, head_group_mask, (hipStream_t)stream));
}

int dsa_sparse_prefill_grouped_varlen(const uint16_t* q, const uint16_t* kv_cache, const float* kv_row_scale,
                                      int num_slots,
                                      const int32_t* group_info, int max_groups, const int32_t* union_idx,
                                      const int32_t* union_len, const uint8_t* head_group_mask, int T,
                                      int H, int union_pad, int d_qk, int d_v, float scale,
                                      uint16_t* out, float* lse, void* stream) {
  if (H != 16 && H != 32 && H != 64 && H != 128) return DSA_ERR_UNSUPPORTED;
  if (!latent_ok(d_qk, d_v) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (T < 0 || num_slots < 1 || max_groups < 0 || union_pad < 0 || union_pad % 32 != 0)
    return DSA_ERR_SHAPE;
  if (T == 0 || max_groups == 0) return DSA_OK;
  if (!q || !kv_cache || !group_info || !union_idx || !union_len || !head_group_mask || !out || !lse)
    return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(kv_cache, 16) || !aligned_to(out, 16) || !aligned_to(lse, 4) ||
      !aligned_to(group_info, 8) || !aligned_to(union_idx, 4) || !aligned_to(union_len, 4) ||
      !aligned_to(head_group_mask, 4) || !aligned_to(kv_row_scale, 4))
    return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_grouped_attn(q, kv_cache, union_idx, union_len, head_group_mask, T, H,
                                                num_slots, union_pad, scale, out, lse, (hipStream_t)stream,
                                                group_info, max_groups, d_qk, kv_row_scale, 1));
}

int dsa_sparse_prefill_pertoken_varlen(const uint16_t* q, const uint16_t* kv_cache, const float* kv_row_scale,
                                       int num_slots,
                                       const int32_t* topk, int64_t ld, int T, int H, int cols, int R,
                                       const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                       const int32_t* q_pos_start, const int32_t* block_table,
                                       int64_t bt_ld, int page_size, int d_qk, int d_v, float scale,
                                       int32_t* topk_ws, uint16_t* out, float* lse, void* stream) {
  if (H < 16 || H > 128 || H % 16 != 0) return DSA_ERR_UNSUPPORTED;
  if (!latent_ok(d_qk, d_v) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (!batch_shape_ok(T, cols, ld, R, bt_ld, page_size, num_slots)) return DSA_ERR_SHAPE;
  if (T == 0) return DSA_OK;
  if (!q || !kv_cache || !out || !lse || (cols > 0 && (!topk || !topk_ws)) ||
      !batch_ptrs_ok(cu_seqlens_q, kv_lens, q_pos_start, block_table))
    return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(kv_cache, 16) || !aligned_to(out, 16) || !aligned_to(lse, 4) ||
      !aligned_to(topk, 4) || !aligned_to(topk_ws, 4) || !aligned_to(kv_row_scale, 4) ||
      !batch_aligned(cu_seqlens_q, kv_lens, q_pos_start, block_table))
    return DSA_ERR_ALIGN;
  // physical-row top-k (causality applied), then the single-sequence kernel over the whole
  // cache with every row in its causal range
  hipError_t e = dsa::launch_convert_req_index(topk, ld, T, cols, R, cu_seqlens_q, kv_lens, q_pos_start,
                                               block_table, bt_ld, page_size, num_slots, topk_ws,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return DSA_ERR_LAUNCH;
  const int64_t all_causal = (int64_t)num_slots - 1;
  if (H == 128)
    e = dsa::launch_pertoken_rows128(q, kv_cache, topk_ws, cols, T, num_slots, cols, all_causal, scale, out,
                                     lse, (hipStream_t)stream, d_qk, kv_row_scale, 1);
  else
    e = dsa::launch_pertoken_attn(q, kv_cache, topk_ws, cols, T, H, num_slots, cols, all_causal, scale, out,
                                  lse, (hipStream_t)stream, d_qk, kv_row_scale, 1);
  return launch_status(e);
}

int dsa_decode_paged_fp8(const uint8_t* cache8, const float* kv_scale, int scale_per_row, int num_slots,
                         int d, int R, const int32_t* kv_lens, const int32_t* block_table, int64_t bt_ld,
                         int page_size, int ws_pages, uint16_t* ws_cache, float* ws_row_scale,
                         int32_t* ws_block_table, void* stream) {
  if (d != 576 && d != 512) return DSA_ERR_UNSUPPORTED;
  if (num_slots < 1 || R < 1 || bt_ld < 1 || page_size < 1 || num_slots % page_size != 0 || ws_pages < 0 ||
      bt_ld > 65535 || R > 65535)
    return DSA_ERR_SHAPE;
  if (!kv_lens || !block_table || !ws_block_table || !ws_row_scale) return DSA_ERR_NULL;
  if (!aligned_to(kv_lens, 4) || !aligned_to(block_table, 4) || !aligned_to(ws_block_table, 4) ||
      !aligned_to(ws_row_scale, 4))
    return DSA_ERR_ALIGN;
  const int st = fp8_check(cache8, kv_scale, scale_per_row, ws_cache);
  if (st != DSA_OK) return st;
  return launch_status(dsa::launch_decode_paged_fp8(cache8, kv_scale, scale_per_row, num_slots, d, R, kv_lens,
                                                    block_table, bt_ld, page_size, ws_pages, ws_cache,
                                                    ws_row_scale, ws_block_table, (hipStream_t)stream));
}

// Host checks of the masked MHA calls (mask_ws is checked only when `with_ws`): DSA_OK when
// the call has work to enqueue, kNothingToDo for an empty one, else the status.
static int masked_check(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe, const uint16_t* v,
                        const int32_t* topk, int64_t ld, int T, int S, int H, int dn, int dr, int dv, int cols,
                        int64_t q_pos_offset, float scale, bool with_ws, const uint32_t* mask_ws,
                        const uint16_t* out, const float* lse) {
  // geometries: NoPE (256, 0, 256), the key is k_nope itself; (192, 64, 256) and
  // (128, 64, 128), the key is k_nope || k_pe with k_pe shared by every head
  const bool nope = mha_nope(dn, dr, dv), rope = mha_rope(dn, dr, dv);
  if ((!nope && !rope) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  // (H <= 65536 keeps the kernels' 32-bit per-lane key-row offsets and the grid in range)
  if (H < 1 || H > 65536 || T < 0 || S < 1 || cols < 0 || ld < cols || q_pos_offset < 0) return DSA_ERR_SHAPE;
  if (((int64_t)T + 255) / 256 * H > 0x7fffffff) return DSA_ERR_SHAPE;  // one workgroup per (256 tokens, head)
  if (T == 0) return kNothingToDo;
  if (!q || !k_nope || !v || (cols > 0 && !topk) || (with_ws && !mask_ws) || !out || !lse || (rope && !k_pe))
    return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(k_nope, 16) || !aligned_to(v, 16) ||
      !aligned_to(out, 16) || !aligned_to(lse, 4) || (with_ws && !aligned_to(mask_ws, 4)) ||
      !aligned_to(topk, 4) || (rope && !aligned_to(k_pe, 16)))
    return DSA_ERR_ALIGN;
  return DSA_OK;
}

static int masked_launch(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe, const uint16_t* v,
                         const int32_t* topk, int64_t ld, int T, int S, int H, int dn, int dr, int dv, int cols,
                         int64_t q_pos_offset, float scale, uint32_t* mask_ws, uint16_t* out, float* lse,
                         void* stream) {
  const bool rope = dr > 0;
  const int words = (S + 31) / 32;
  hipError_t e = dsa::launch_scatter_topk_bits(topk, ld, T, cols, S, q_pos_offset, mask_ws, words,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return DSA_ERR_LAUNCH;
  return launch_status(dsa::launch_masked_mha(q, k_nope, rope ? k_pe : nullptr, dn, dr, dv, v, mask_ws,
                                              words, T, S, H, q_pos_offset, scale, out, lse,
                                              (hipStream_t)stream));
}

int dsa_masked_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                           const uint16_t* v, const int32_t* topk, int64_t ld, int T, int S, int H,
                           int dn, int dr, int dv, int cols, int64_t q_pos_offset, float scale,
                           uint32_t* mask_ws, uint16_t* out, float* lse, void* stream) {
  const int st = masked_check(q, k_nope, k_pe, v, topk, ld, T, S, H, dn, dr, dv, cols, q_pos_offset, scale, true,
                              mask_ws, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  return masked_launch(q, k_nope, k_pe, v, topk, ld, T, S, H, dn, dr, dv, cols, q_pos_offset, scale, mask_ws, out,
                       lse, stream);
}

int dsa_dense_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                          const uint16_t* v, int T, int S, int H, int dn, int dr, int dv,
                          int64_t q_pos_offset, float scale, uint16_t* out, float* lse, void* stream) {
  const bool nope = mha_nope(dn, dr, dv), rope = mha_rope(dn, dr, dv);
  if ((!nope && !rope) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (H < 1 || H > 65536 || T < 0 || S < 1 || q_pos_offset < 0) return DSA_ERR_SHAPE;
  if (((int64_t)T + 255) / 256 * H > 0x7fffffff) return DSA_ERR_SHAPE;  // one workgroup per (256 tokens, head)
  if (T == 0) return DSA_OK;
  if (!q || !k_nope || !v || !out || !lse || (rope && !k_pe)) return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(k_nope, 16) || !aligned_to(v, 16) ||
      !aligned_to(out, 16) || !aligned_to(lse, 4) || (rope && !aligned_to(k_pe, 16)))
    return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_masked_mha(q, k_nope, rope ? k_pe : nullptr, dn, dr, dv, v, nullptr, 0,
                                              T, S, H, q_pos_offset, scale, out, lse, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: the masked-MHA bit mask in a static device array.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchWords = DSA_SCRATCH_BYTES / sizeof(uint32_t);
constexpr int kMaxDevices = 64;
// this array's device address on each GPU, taken once per device with that device current
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

// Per GPU, held until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels get the address hipGetSymbolAddress returns.
static __device__ __align__(256) uint32_t scratch[kScratchWords];

// the device address of `scratch` on the current device (DSA_OK), or DSA_ERR_LAUNCH
static int scratch_address(uint32_t** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_LAUNCH;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // (two threads may both get here first: they store the same address)
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSA_ERR_LAUNCH;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = static_cast<uint32_t*>(p);
  return DSA_OK;
}

extern "C" int dsa_masked_mha_prefill_noalloc(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                                              const uint16_t* v, const int32_t* topk, int64_t ld, int T, int S,
                                              int H, int dn, int dr, int dv, int cols, int64_t q_pos_offset,
                                              float scale, uint16_t* out, float* lse, void* stream) {
  const int st = masked_check(q, k_nope, k_pe, v, topk, ld, T, S, H, dn, dr, dv, cols, q_pos_offset, scale, false,
                              nullptr, out, lse);
  if (st != DSA_OK) return st == kNothingToDo ? DSA_OK : st;
  if (dsa_masked_mha_workspace_bytes(T, S) > DSA_SCRATCH_BYTES) return DSA_ERR_CAPACITY;
  uint32_t* mask_ws = nullptr;
  const int sa = scratch_address(&mask_ws);
  if (sa != DSA_OK) return sa;
  return masked_launch(q, k_nope, k_pe, v, topk, ld, T, S, H, dn, dr, dv, cols, q_pos_offset, scale, mask_ws, out,
                       lse, stream);
}
