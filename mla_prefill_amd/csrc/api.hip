// C-ABI host layer of libdsa_prefill.so: argument checks, then kernel launches
// on the caller's stream.  Nothing here allocates, frees or synchronizes.
#include <limits.h>
#include <stdint.h>

#include "dsa_prefill.h"
#include "kernels.h"

namespace {

inline bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

// the kernels fold the scale into exponent FMAs on raw scores: it must be finite and nonzero
inline bool scale_ok(float s) { return s == s && s != 0.f && s - s == 0.f; }

constexpr int kLatentDim = 576;
constexpr int kValueDim = 512;

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
    default: return "unknown status";
  }
}

int dsa_union_pad(int G, int cols) {
  if (G < 1 || G > 8 || cols < 0) return DSA_ERR_SHAPE;
  const long long v = ((long long)G * cols + 63) / 64 * 64;
  if (v > INT_MAX) return DSA_ERR_SHAPE;
  return (int)v;
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

int dsa_sparse_prefill_grouped(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                               const int32_t* union_len, const uint8_t* head_group_mask, int T,
                               int H, int S, int union_pad, int d_qk, int d_v, float scale,
                               uint16_t* out, float* lse, void* stream) {
  if (H != 16 && H != 32 && H != 64 && H != 128) return DSA_ERR_UNSUPPORTED;
  if (d_qk != kLatentDim || d_v != kValueDim || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (T < 0 || S < 1 || union_pad < 0 || union_pad % 32 != 0) return DSA_ERR_SHAPE;
  if (T == 0) return DSA_OK;
  if (!q || !kv || !union_idx || !union_len || !head_group_mask || !out || !lse)
    return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(kv, 16) || !aligned_to(out, 16) || !aligned_to(lse, 4) ||
      !aligned_to(union_idx, 4) || !aligned_to(union_len, 4) || !aligned_to(head_group_mask, 4))
    return DSA_ERR_ALIGN;
  return launch_status(dsa::launch_grouped_attn(q, kv, union_idx, union_len, head_group_mask, T,
                                                H, S, union_pad, scale, out, lse,
                                                (hipStream_t)stream));
}

int dsa_sparse_prefill_pertoken(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                int d_qk, int d_v, float scale, uint16_t* out, float* lse,
                                void* stream) {
  if (H < 16 || H > 128 || H % 16 != 0) return DSA_ERR_UNSUPPORTED;
  if (d_qk != kLatentDim || d_v != kValueDim || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (T < 0 || S < 1 || cols < 0 || ld < cols || q_pos_offset < 0) return DSA_ERR_SHAPE;
  if (T == 0) return DSA_OK;
  if (!q || !kv || (cols > 0 && !topk) || !out || !lse) return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(kv, 16) || !aligned_to(out, 16) || !aligned_to(lse, 4) ||
      !aligned_to(topk, 4))
    return DSA_ERR_ALIGN;
  hipError_t e;
  if (H == 128)
    e = dsa::launch_pertoken_rows128(q, kv, topk, ld, T, S, cols, q_pos_offset, scale, out, lse,
                                     (hipStream_t)stream);
  else
    e = dsa::launch_pertoken_attn(q, kv, topk, ld, T, H, S, cols, q_pos_offset, scale, out, lse,
                                  (hipStream_t)stream);
  return launch_status(e);
}

int dsa_masked_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                           const uint16_t* v, const int32_t* topk, int64_t ld, int T, int S, int H,
                           int dn, int dr, int dv, int cols, int64_t q_pos_offset, float scale,
                           uint32_t* mask_ws, uint16_t* out, float* lse, void* stream) {
  // geometries: NoPE (256, 0, 256), the key is k_nope itself; (192, 64, 256), the key is
  // k_nope || k_pe with k_pe shared by every head
  const bool nope = dn == 256 && dr == 0 && dv == 256;
  const bool rope = dn == 192 && dr == 64 && dv == 256;
  if ((!nope && !rope) || !scale_ok(scale)) return DSA_ERR_UNSUPPORTED;
  if (H < 1 || T < 0 || S < 1 || cols < 0 || ld < cols || q_pos_offset < 0) return DSA_ERR_SHAPE;
  if (T == 0) return DSA_OK;
  if (!q || !k_nope || !v || (cols > 0 && !topk) || !mask_ws || !out || !lse || (rope && !k_pe))
    return DSA_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(k_nope, 16) || !aligned_to(v, 16) ||
      !aligned_to(out, 16) || !aligned_to(lse, 4) || !aligned_to(mask_ws, 4) ||
      !aligned_to(topk, 4) || (rope && !aligned_to(k_pe, 16)))
    return DSA_ERR_ALIGN;
  const int words = (S + 31) / 32;
  hipError_t e = dsa::launch_scatter_topk_bits(topk, ld, T, cols, S, q_pos_offset, mask_ws, words,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return DSA_ERR_LAUNCH;
  return launch_status(dsa::launch_masked_mha(q, k_nope, rope ? k_pe : nullptr, dn, v, mask_ws, words, T,
                                              S, H, q_pos_offset, scale, out, lse,
                                              (hipStream_t)stream));
}

}  // extern "C"
