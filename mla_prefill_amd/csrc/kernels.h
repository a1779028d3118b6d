// Internal launchers of the HIP kernels (called by the C-ABI layer in api.cpp
// after it has validated every argument).  Each enqueues on `stream`, never
// allocates, never synchronizes, and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

hipError_t launch_build_union(const int32_t* topk, int64_t ld, int T, int cols, int S,
                              int64_t q_pos_offset, int G, int union_pad, int32_t* union_idx,
                              int32_t* union_len, uint8_t* head_group_mask, hipStream_t stream);

// A batch of requests over a paged cache: union/mask per group of consecutive tokens of
// one request (groups numbered request by request; group_info[g] = first token, count),
// list entries written as physical rows.
hipError_t launch_build_union_varlen(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                     const int32_t* cu_seqlens, const int32_t* kv_lens,
                                     const int32_t* q_pos_start, const int32_t* block_table,
                                     int64_t bt_ld, int page_size, int num_slots, int G, int max_groups,
                                     int union_pad, int32_t* group_info, int32_t* union_idx,
                                     int32_t* union_len, uint8_t* head_group_mask, hipStream_t stream);
// request-local top-k entries -> physical rows (-1: selects nothing), out [T, cols]
hipError_t launch_convert_req_index(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                    const int32_t* cu_seqlens, const int32_t* kv_lens,
                                    const int32_t* q_pos_start, const int32_t* block_table, int64_t bt_ld,
                                    int page_size, int num_slots, int32_t* out, hipStream_t stream);

hipError_t launch_scatter_topk_bits(const int32_t* topk, int64_t ld, int T, int cols, int S,
                                    int64_t q_pos_offset, uint32_t* bits, int words,
                                    hipStream_t stream);

// Row scales of the latent (every MQA launcher): kscale == nullptr for a plain bf16 latent;
// otherwise row x's elements are its bf16 values times kscale[scale_per_row ? x : 0] (an FP8
// latent decoded exactly to bf16): the kernels scale each key's raw score and each
// probability before the PV product by it.

// `skip` (optional, device): when *skip != 0 at run time the attention kernels return at
// once -- the routing chosen on the device by launch_route_by_union (route[0] gates the
// grouped kernels, route[1] the per-token kernel).
hipError_t launch_route_by_union(const int32_t* union_len, int NG, int union_pad, double limit, int32_t* route,
                                 hipStream_t stream);

// per-token sparse MQA for H % 16 == 0 (one workgroup per (token, 16-head block))
hipError_t launch_pertoken_attn(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                float scale, uint16_t* out, float* lse, hipStream_t stream, int d_qk,
                                const float* kscale = nullptr, int scale_per_row = 0,
                                const int32_t* skip = nullptr);

// 128-row attention over a per-workgroup key list.  Grouped mode: rows are the
// 128 pseudo-heads of a group, keys the group's union list, and each row is
// restricted by its token's bit of head_group_mask.  Per-token mode (H = 128):
// rows are the token's heads and keys its top-k row.  group_info (nullptr: group g is
// tokens gG ..) gives each of max_groups groups' first token and token count.
hipError_t launch_grouped_attn(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                               const int32_t* union_len, const uint8_t* head_group_mask, int T,
                               int H, int S, int union_pad, float scale, uint16_t* out, float* lse,
                               hipStream_t stream, const int32_t* group_info, int max_groups, int d_qk,
                               const float* kscale = nullptr, int scale_per_row = 0,
                               const int32_t* skip = nullptr);
hipError_t launch_pertoken_rows128(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                   int64_t ld, int T, int S, int cols, int64_t q_pos_offset,
                                   float scale, uint16_t* out, float* lse, hipStream_t stream, int d_qk,
                                   const float* kscale = nullptr, int scale_per_row = 0);

// The fast 128-row kernel fixes each row's softmax reference at the row's first valid
// scores.  A group in which a later score exceeds that reference by more than 2^64 gets
// this NaN bit pattern in the LSE of all its rows; launch_rows128_exact then recomputes
// exactly those groups with a running-max softmax (other workgroups return at once).
// hgmask == nullptr selects the per-token mode.
constexpr uint32_t kOverflowMark = 0x7fa5a5a5u;
hipError_t launch_rows128_exact(const uint16_t* q, const uint16_t* kv, const int32_t* keys,
                                int64_t keys_ld, const int32_t* union_len, const uint8_t* hgmask,
                                int T, int H, int S, int ncols, int64_t q_pos_offset, float scale,
                                uint16_t* out, float* lse, hipStream_t stream, const int32_t* group_info,
                                int ngroups, int d_qk, const float* kscale, int scale_per_row,
                                const int32_t* skip = nullptr);

// FP8 (OCP E4M3) codes -> the bf16 numbers they encode (exact; no scale applied); rows x d
// codes, d a multiple of 16
hipError_t launch_decode_fp8(const uint8_t* kv8, int64_t rows, int d, uint16_t* out, hipStream_t stream);
// a batch over a paged FP8 cache: each request's reachable pages decoded into a compact bf16
// workspace of ws_pages pages, each workspace row's scale, and the block table over it (-1
// where nothing maps)
hipError_t launch_decode_paged_fp8(const uint8_t* cache8, const float* scale, int per_row, int num_slots, int d,
                                   int R, const int32_t* kv_lens, const int32_t* block_table, int64_t bt_ld,
                                   int page_size, int ws_pages, uint16_t* out_cache, float* out_scale,
                                   int32_t* out_bt, hipStream_t stream);

// masked dense MHA, key = k_nope (dn) + shared k_pe (dr), value dv: (256, 0, 256),
// (192, 64, 256) or (128, 64, 128); mask = causal AND top-k bit; bits == nullptr: causal
// only (dense MHA)
hipError_t launch_masked_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe, int dn,
                             int dr, int dv, const uint16_t* v, const uint32_t* bits, int words, int T,
                             int S, int H, int64_t q_pos_offset, float scale, uint16_t* out, float* lse,
                             hipStream_t stream);

}  // namespace dsa
