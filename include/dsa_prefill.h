/*
 * dsa_prefill.h -- C ABI of libdsa_prefill.so: DSA sparse-MLA prefill attention
 * on AMD Instinct MI355X (gfx950).
 *
 * Every query token attends only over its own indexer-selected top-k KV rows;
 * the result is per-token sparse softmax attention, out plus LSE.  The pages
 * describe three routings of this one function, each exposed here:
 *
 *   per-token  -- dsa_sparse_prefill_pertoken: each token gathers its own rows
 *                 of the bf16 latent ("[Perf][GLM-5.3-Flash]
 *                 Dense/masked-MHA sparse prefill for the NoPE (256, 0, 256)
 *                 layout + skip the NoPE K concat", Purpose section);
 *   grouped    -- dsa_build_group_union + dsa_sparse_prefill_grouped: 128/H
 *                 consecutive tokens become 128 pseudo-heads over the sorted
 *                 union of their top-k sets, with a per-token membership mask
 *                 ("[Perf][DSA] Grouped sparse prefill with the FlashMLA
 *                 head-group-mask kernel", commit message and "How" section);
 *   masked MHA -- dsa_masked_mha_prefill: dense MHA with mask = causal AND
 *                 top-k membership ("[2/N][Attention] Enable masked MHA for
 *                 sparse MLA prefills", Purpose section); its mask-free
 *                 special case for chunks no longer than the top-k is
 *                 dsa_dense_mha_prefill.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - All tensor pointers are DEVICE pointers owned by the caller.  Tensors are
 *    contiguous row-major; the top-k buffer alone has a leading dimension `ld`
 *    (int32 elements between consecutive token rows, ld >= cols).
 *  - bf16 tensors must be 16-byte aligned; int32 / float tensors 4-byte
 *    aligned.  Outputs must not alias inputs.
 *  - The library never allocates, frees or synchronizes.  All work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *    completes asynchronously.
 *  - Selection rule, identical in every routing: token t (at absolute position
 *    p_t = q_pos_offset + t) selects entry x of its top-k row iff 0 <= x < S and
 *    x <= p_t.  -1 padding, out-of-range and non-causal entries are ignored, so
 *    kernels stay memory-safe for any index contents.  Valid entries of a row
 *    must be distinct (a top-k is a set); with duplicates the union list and
 *    masks stay well defined but per-token results are unspecified.
 *  - A token that selects nothing gets out = 0 and lse = -inf.
 *  - out is bf16 (round to nearest even) of the fp32 result; lse is fp32, the
 *    natural log of the sum of exp(scale * q.k) over the token's selection.
 *  - scale must be finite and nonzero (either sign); other values are
 *    rejected with DSA_ERR_UNSUPPORTED.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    rejected call enqueues nothing and returns a negative status.
 */
#ifndef DSA_PREFILL_H
#define DSA_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2

/* status codes */
#define DSA_OK 0
#define DSA_ERR_NULL (-1)        /* a required pointer is NULL */
#define DSA_ERR_SHAPE (-2)       /* a size or leading dimension is out of range */
#define DSA_ERR_UNSUPPORTED (-3) /* head count / head dims / scale outside the supported set */
#define DSA_ERR_ALIGN (-4)       /* a pointer is not aligned as required */
#define DSA_ERR_LAUNCH (-5)      /* the HIP runtime rejected a kernel launch */
#define DSA_ERR_CAPACITY (-6)    /* the work needs more than the library's static scratch */

/* Version of this ABI (DSA_ABI_VERSION). */
int dsa_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* dsa_status_string(int status);

/* Padded length of one group's union list: ceil(G * cols / 64) * 64 (the
 * pages pad the union to whole blocks; block = 64 here).  Returns
 * DSA_ERR_SHAPE for G outside 1..8, cols < 0 or an int overflow. */
int dsa_union_pad(int G, int cols);

/* Bytes of the bit-packed masked-MHA workspace: T * ceil(S / 32) * 4
 * (0 for negative sizes). */
size_t dsa_masked_mha_workspace_bytes(int T, int S);

/* Routing of one chunk on MI355X ("[2/N][Attention] Enable masked MHA for
 * sparse MLA prefills", Purpose section and its heuristic commit: a masked
 * MHA beats the sparse MQA kernels below some sequence length, and a chunk
 * whose tokens' top-k hold every causal key is plain causal attention).
 *   T, S, q_pos_offset  the chunk: T query tokens at positions
 *                       q_pos_offset .. q_pos_offset + T - 1 over S keys
 *   H                   query heads on this GPU
 *   k                   the indexer's top-k size
 *   mha_dv              the value width of the caller's per-head MHA geometry
 *                       when it can run the MHA forms: 256 for (256, 0, 256)
 *                       and (192, 64, 256), 128 for (128, 64, 128); 0 when it
 *                       cannot (the choice is then grouped or per-token)
 * Returns one of the DSA_ROUTING_* codes:
 *   DENSE     mha_dv != 0 and q_pos_offset + T <= k;
 *   MASKED    mha_dv != 0 and the mean over the chunk of the causal key count
 *             min(S, p_t + 1) is at most c * k, with c measured on MI355X for
 *             this library's kernels (against the 576-wide latent):
 *                         H = 16   32   64  | 128 | other multiples of 16
 *               mha_dv 256:  2.4  1.95 1.7  | 1.4 | 3.4
 *               mha_dv 128:  3.6  3.05 2.75 | 2.4 | 5.5
 *             (first three against grouped, the rest against per-token); any
 *             H the MQA kernels do not take (not a multiple of 16, or above
 *             128) routes here as well;
 *   GROUPED   H in {16, 32, 64} (128 / H consecutive tokens per group);
 *   PERTOKEN  otherwise (H = 128 runs per-token: a group would be one token).
 * DSA_ERR_SHAPE for T < 0, S < 1, q_pos_offset < 0, H < 1 or k < 1;
 * DSA_ERR_UNSUPPORTED for another mha_dv, or when no routing serves H (MQA
 * kernels need H a multiple of 16 up to 128, and mha_dv is 0).  Host-only:
 * nothing is enqueued. */
#define DSA_ROUTING_DENSE 1
#define DSA_ROUTING_MASKED 2
#define DSA_ROUTING_GROUPED 3
#define DSA_ROUTING_PERTOKEN 4
int dsa_select_routing(int T, int S, int64_t q_pos_offset, int H, int k, int mha_dv);

/* Union list and per-token membership mask of every group of G consecutive
 * tokens ("[Perf][DSA] Grouped sparse prefill ...", "How" section: sorted
 * union by bitmap and prefix sum, per-token membership mask).
 *
 *   topk            int32 [T, ld], first `cols` entries of each row used
 *   T, cols, S      query tokens, top-k columns used, KV rows (T >= 0, cols >= 0, S >= 1)
 *   q_pos_offset    position of token 0 (>= 0); token t sits at q_pos_offset + t
 *   G               tokens per group, 1..8 (128 / H for the grouped routing)
 *   union_pad       row length of the outputs; a multiple of 64 and >= G * cols
 *                   (dsa_union_pad(G, cols) is the smallest such value)
 * Outputs, NG = ceil(T / G) groups, group g = tokens gG .. min(T, gG + G) - 1:
 *   union_idx       int32 [NG, union_pad]: the strictly ascending union of the
 *                   members' selections, then -1 up to the next multiple of 64
 *                   (entries past that are not written)
 *   union_len       int32 [NG]: number of union entries
 *   head_group_mask uint8 [NG, union_pad]: bit i of slot j is set iff token
 *                   gG + i selects union_idx[g, j]; 0 in the written padding
 *                   slots and for absent members of the last group.
 * union_len and each row's slots up to the next multiple of 64 past its union are
 * written (the attention kernels read no further).  Bit-exact and deterministic. */
int dsa_build_group_union(const int32_t* topk, int64_t ld, int T, int cols, int S,
                          int64_t q_pos_offset, int G, int union_pad, int32_t* union_idx,
                          int32_t* union_len, uint8_t* head_group_mask, void* stream);

/* Grouped sparse attention ("[Perf][DSA] Grouped sparse prefill ...", commit
 * message and "How" section): with G = 128 / H, row r = i * H + h of group g
 * (token gG + i, head h) attends over the slots j < union_len[g] of
 * union_idx[g] whose mask bit i is set; this equals per-token attention.
 *
 *   q         bf16 [T, H, d_qk] absorbed MLA queries (free view [NG, 128, d_qk])
 *   kv        bf16 [S, d_qk] latent rows; V = the first 512 dims of a row
 *   union_idx, union_len, head_group_mask: as written by dsa_build_group_union
 *             (union_len is clamped to [0, union_pad]; slots holding a
 *             position outside [0, S) are skipped); union_pad must be a
 *             multiple of 32 (dsa_union_pad gives a multiple of 64) and
 *             head_group_mask 4-byte aligned
 *   H         16, 32, 64 or 128 (128 % H == 0 and G = 128 / H <= 8)
 *   d_qk      576 (512 latent dims + 64 rope dims) or 512 (the GLM-5.3-Flash
 *             latent with no rope part, "[Perf][GLM-5.3-Flash] ...": scores
 *             and values then use the same 512 dims); d_v must be 512
 *   scale     softmax scale applied to q.k
 *   out       bf16 [T, H, 512];  lse  fp32 [T, H]
 * Rows of the partial last group beyond T are neither read nor written. */
int dsa_sparse_prefill_grouped(const uint16_t* q, const uint16_t* kv, const int32_t* union_idx,
                               const int32_t* union_len, const uint8_t* head_group_mask, int T,
                               int H, int S, int union_pad, int d_qk, int d_v, float scale,
                               uint16_t* out, float* lse, void* stream);

/* Sparse MQA prefill with the routing chosen on the device from the union's
 * size (grouped and per-token forms as above; both compute per-token attention,
 * "[Perf][DSA] Grouped sparse prefill ...", "How" section).  The union and
 * membership mask of every group of G = 128 / H tokens are built; then one
 * workgroup sums the grouped form's tiles, ceil(union_len / 32) over the groups,
 * and compares them with the per-token form's cost in the same unit,
 * rho(H) * sum_t min(cols, S, q_pos_offset + t + 1) / 32 with rho = 0.22, 0.46,
 * 0.94 for H = 16, 32, 64 (measured on MI355X for this library's kernels).
 * Both attention launches are enqueued; the one not chosen returns at once.
 *
 *   q, kv, topk, ld, T, H, S, cols, q_pos_offset, d_qk, d_v, scale, out, lse:
 *             as for dsa_sparse_prefill_pertoken; H must be 16, 32 or 64
 *   union_pad, union_idx, union_len, head_group_mask: the union workspace, as
 *             for dsa_build_group_union with G = 128 / H (overwritten)
 *   route     int32 [4] device workspace (overwritten, 4-byte aligned): after
 *             the call route[0] = 1 if the per-token form ran (grouped
 *             skipped), route[1] = 1 if the grouped form ran, route[2] = the
 *             union's tile count (saturated at 2^31 - 1); route[3] is unused
 * Errors as for the grouped and per-token calls; DSA_ERR_UNSUPPORTED for another H.
 * The result equals either form's (within its rounding). */
int dsa_sparse_prefill_auto(const uint16_t* q, const uint16_t* kv, const int32_t* topk, int64_t ld, int T,
                            int H, int S, int cols, int64_t q_pos_offset, int d_qk, int d_v, float scale,
                            int union_pad, int32_t* union_idx, int32_t* union_len, uint8_t* head_group_mask,
                            int32_t* route, uint16_t* out, float* lse, void* stream);

/* Per-token sparse MQA ("[Perf][GLM-5.3-Flash] ...", Purpose section): token t
 * attends, for each head, over the latent rows it selects from its own top-k
 * row (selection rule above), gathering them itself.
 *
 *   q [T, H, d_qk], kv [S, d_qk], topk int32 [T, ld] (cols used), H a multiple
 *   of 16 up to 128, d_qk = 576 or 512 (as for the grouped form), d_v = 512,
 *   q_pos_offset >= 0;
 *   out bf16 [T, H, 512], lse fp32 [T, H]. */
int dsa_sparse_prefill_pertoken(const uint16_t* q, const uint16_t* kv, const int32_t* topk,
                                int64_t ld, int T, int H, int S, int cols, int64_t q_pos_offset,
                                int d_qk, int d_v, float scale, uint16_t* out, float* lse,
                                void* stream);

/* Masked dense MHA ("[2/N][Attention] Enable masked MHA for sparse MLA
 * prefills", Purpose section; "[Perf][GLM-5.3-Flash] ...", commit messages):
 * token t, head h attends over every key x with x <= q_pos_offset + t and
 * x in sel(t), using per-head keys and values.  Supported geometries (the
 * three (qk_nope, qk_rope, v) tuples of the pages' masked-MHA allow-list,
 * "[Perf][GLM-5.3-Flash] ..." description and commit messages):
 *   dn = 256, dr = 0,  dv = 256 (NoPE): the key is k_nope itself, read in
 *     place; k_pe is not read (it may be NULL);
 *   dn = 192, dr = 64, dv = 256 (GLM-5) and dn = 128, dr = 64, dv = 128
 *   (DeepSeek-V3.2): the key is k_nope || k_pe, k_pe shared by every head (the
 *   broadcast the pages' K concat builds); both are read in place, no
 *   concatenated K is materialized.  k_pe must be non-NULL and 16-byte
 *   aligned.
 * Anything else returns DSA_ERR_UNSUPPORTED.
 *
 *   q       bf16 [T, H, dn + dr];  k_nope bf16 [S, H, dn];  k_pe bf16 [S, dr]
 *   v       bf16 [S, H, dv]
 *   topk    int32 [T, ld] (cols used)
 *   mask_ws uint32 [T, ceil(S / 32)] caller-owned workspace of
 *           dsa_masked_mha_workspace_bytes(T, S) bytes; overwritten with the
 *           bit-packed top-k membership (bit x % 32 of word x / 32 of row t)
 *   out     bf16 [T, H, dv];  lse fp32 [T, H]
 *   H       1 .. 65536, and ceil(T / 256) * H < 2^31 (else DSA_ERR_SHAPE)
 * Three kernels are enqueued: the mask scatter, the attention, and an exact
 * pass that returns at once unless a row's scores rose more than 2^64 above
 * the attention kernel's fixed softmax reference (it then recomputes that
 * row's 256-token tile with a running max). */
int dsa_masked_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                           const uint16_t* v, const int32_t* topk, int64_t ld, int T, int S, int H,
                           int dn, int dr, int dv, int cols, int64_t q_pos_offset, float scale,
                           uint32_t* mask_ws, uint16_t* out, float* lse, void* stream);

/* For callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): dsa_masked_mha_prefill without the
 * mask_ws argument.  The bit-packed top-k mask lives in a static device array
 * of the library, DSA_SCRATCH_BYTES on each GPU it runs on, held until the
 * process ends; the call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine) and does not synchronize.  Every call on a GPU
 * shares that GPU's array, and each call rewrites the T * ceil(S / 32) words
 * it uses before reading them, so calls that overlap on one GPU (on other
 * streams or threads) race and must be ordered by the caller.
 * DSA_ERR_CAPACITY when dsa_masked_mha_workspace_bytes(T, S) exceeds
 * DSA_SCRATCH_BYTES (e.g. T = S = 16384 fits; T = 16384, S = 32800 does not);
 * DSA_ERR_LAUNCH also when the array's device address cannot be obtained.
 * Every other argument, check and result as dsa_masked_mha_prefill. */
#define DSA_SCRATCH_BYTES ((size_t)32 << 20)
int dsa_masked_mha_prefill_noalloc(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                                   const uint16_t* v, const int32_t* topk, int64_t ld, int T, int S, int H,
                                   int dn, int dr, int dv, int cols, int64_t q_pos_offset, float scale,
                                   uint16_t* out, float* lse, void* stream);

/* Dense causal MHA, the shortcut for chunks no longer than the top-k ("[2/N]
 * [Attention] Enable masked MHA for sparse MLA prefills", Purpose section:
 * when every causal key is among a token's top-k, the selection is the causal
 * mask and sparse attention is plain causal attention).  Token t, head h
 * attends over every key x <= q_pos_offset + t (x < S).  It equals
 * dsa_masked_mha_prefill whenever each token's top-k row holds all of its
 * causal positions, i.e. whenever q_pos_offset + T <= the top-k size; the
 * caller decides when that holds -- no top-k is read here.  Geometries,
 * layouts, alignment and errors as dsa_masked_mha_prefill (without topk and
 * mask_ws).  Two kernels are enqueued: the attention and the exact pass
 * described there. */
int dsa_dense_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_pe,
                          const uint16_t* v, int T, int S, int H, int dn, int dr, int dv,
                          int64_t q_pos_offset, float scale, uint16_t* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 KV latent.  The pages gate quantized KV caches off the grouped path
 * ("[Perf][DSA] Grouped sparse prefill ...", "How" section) and give no FP8
 * format; this library takes OCP E4M3 codes (uint8; sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals, S.1111.111 = NaN) and float32 scales:
 * element (x, i) = e4m3(kv8[x, i]) * kv_scale[scale_per_row ? x : 0], and the
 * attention is the bf16 definition above on those exact values.
 * Every E4M3 value is a bf16 number, so each latent row is decoded once per
 * call, without rounding, into a caller workspace of bf16 rows (no scale
 * applied); the attention kernels then multiply each key's score and each
 * probability by the key row's scale (finite scales; l and the LSE use the
 * unscaled probabilities).  A row is gathered about T * k / S times per chunk,
 * so one decode per row is far cheaper than one per use.
 *   kv8       uint8 [S, d] codes, 16-byte aligned;  kv_scale float32 [S] or [1]
 *   scale_per_row  1: kv_scale[x] for row x;  0: kv_scale[0] for every row
 *   kv_ws     bf16 [S, d] workspace (16-byte aligned), overwritten
 * --------------------------------------------------------------------------- */

/* Decode FP8 codes (d = 576 or 512 per row) to the bf16 numbers they encode:
 * out[x, i] = e4m3(kv8[x, i]), exactly; no scale is applied.  One kernel is
 * enqueued. */
int dsa_decode_latent_fp8(const uint8_t* kv8, int S, int d, uint16_t* out, void* stream);

/* dsa_sparse_prefill_grouped over an FP8 latent: the decode into kv_ws, then
 * grouped attention over kv_ws with the row scales.  Arguments and errors as
 * the bf16 form plus the FP8 ones above; every check precedes the first
 * enqueue. */
int dsa_sparse_prefill_grouped_fp8(const uint16_t* q, const uint8_t* kv8, const float* kv_scale,
                                   int scale_per_row, const int32_t* union_idx, const int32_t* union_len,
                                   const uint8_t* head_group_mask, int T, int H, int S, int union_pad,
                                   int d_qk, int d_v, float scale, uint16_t* kv_ws, uint16_t* out, float* lse,
                                   void* stream);

/* dsa_sparse_prefill_pertoken over an FP8 latent (decode, then the per-token
 * path with the row scales), as dsa_sparse_prefill_grouped_fp8. */
int dsa_sparse_prefill_pertoken_fp8(const uint16_t* q, const uint8_t* kv8, const float* kv_scale,
                                    int scale_per_row, const int32_t* topk, int64_t ld, int T, int H, int S,
                                    int cols, int64_t q_pos_offset, int d_qk, int d_v, float scale,
                                    uint16_t* kv_ws, uint16_t* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Batches of requests over a paged KV cache ("[Perf][DSA] Grouped sparse
 * prefill ...", "How" section: groups are consecutive tokens of one request,
 * and the union's request-local positions become physical rows through the
 * request's index conversion before the attention).
 *
 * A batch of R >= 1 requests is described by device arrays:
 *   cu_seqlens_q int32 [R + 1]  query tokens of request r are cu[r] .. cu[r+1]-1
 *                               (ascending, cu[0] = 0, cu[R] = T)
 *   kv_lens      int32 [R]      request r has positions 0 .. kv_lens[r] - 1
 *   q_pos_start  int32 [R]      position of request r's first query token
 *   block_table  int32 [R, bt_ld]  physical page of each request page: position
 *                               x lives in cache row block_table[r][x / page_size]
 *                               * page_size + x % page_size
 *   page_size >= 1; the cache holds num_slots >= 1 rows of d_qk bf16 (576 or
 *   512, as for the single-sequence forms).
 * Top-k rows hold request-local positions.  Token t of request r (local index
 * i = t - cu[r], position p = q_pos_start[r] + i) selects x iff 0 <= x <
 * kv_lens[r], x <= p and x maps to a row inside the cache (a page past bt_ld or
 * a negative page id maps nowhere).  These contents are data, never errors: any
 * values are memory-safe.  The host checks only sizes, pointers and alignment.
 * ------------------------------------------------------------------------- */

/* Upper bound on a batch's group count, min(T, ceil(T / G) + R): each request
 * adds at most one partial group.  DSA_ERR_SHAPE for T < 0, R < 1 or G outside
 * 1..8. */
int dsa_varlen_group_bound(int T, int R, int G);

/* The index conversion: topk_global int32 [T, cols] (contiguous) receives, for
 * each top-k entry, the cache row it selects, or -1 where it selects nothing. */
int dsa_convert_req_index_to_global(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                    const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                    const int32_t* q_pos_start, const int32_t* block_table, int64_t bt_ld,
                                    int page_size, int num_slots, int32_t* topk_global, void* stream);

/* Union list and membership mask of every group of a batch.  Groups are
 * numbered request by request, ceil(n_r / G) per request, each covering up to G
 * consecutive tokens of one request; max_groups >= the batch's group count
 * (dsa_varlen_group_bound is one such value), later groups are empty.
 *   group_info      int32 [max_groups, 2] (8-byte aligned): first token and token
 *                   count of each group (0, 0 for empty groups)
 *   union_idx       int32 [max_groups, union_pad]: the union of the members'
 *                   selections in ascending request-local position, each written
 *                   as its cache row, then -1 up to the next multiple of 64
 *   union_len, head_group_mask: as for dsa_build_group_union (bit i <-> the
 *                   group's i-th token)
 * group_info and union_len are fully overwritten, union rows as for
 * dsa_build_group_union.  Bit-exact and deterministic. */
int dsa_build_group_union_varlen(const int32_t* topk, int64_t ld, int T, int cols, int R,
                                 const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                 const int32_t* q_pos_start, const int32_t* block_table, int64_t bt_ld,
                                 int page_size, int num_slots, int G, int max_groups, int union_pad,
                                 int32_t* group_info, int32_t* union_idx, int32_t* union_len,
                                 uint8_t* head_group_mask, void* stream);

/* Grouped sparse attention of a batch: as dsa_sparse_prefill_grouped, with
 * group g's tokens taken from group_info (as written by
 * dsa_build_group_union_varlen; entries are clamped into [0, T)) and the keys
 * read from the cache rows union_idx names (rows outside [0, num_slots) are
 * skipped).  Tokens covered by no group are not written.
 *   kv_row_scale  NULL for a bf16 cache; else float32 [num_slots] (4-byte
 *                 aligned), the scale of each cache row, which then holds
 *                 decoded FP8 codes (the workspace dsa_decode_paged_fp8 writes):
 *                 row x's elements are its values times kv_row_scale[x]. */
int dsa_sparse_prefill_grouped_varlen(const uint16_t* q, const uint16_t* kv_cache, const float* kv_row_scale,
                                      int num_slots,
                                      const int32_t* group_info, int max_groups, const int32_t* union_idx,
                                      const int32_t* union_len, const uint8_t* head_group_mask, int T,
                                      int H, int union_pad, int d_qk, int d_v, float scale,
                                      uint16_t* out, float* lse, void* stream);

/* Per-token sparse MQA of a batch: the index conversion into the caller's
 * workspace topk_ws int32 [T, cols], then dsa_sparse_prefill_pertoken over the
 * whole cache with every row in every token's causal range.  Two kernels are
 * enqueued.  kv_row_scale as for dsa_sparse_prefill_grouped_varlen. */
int dsa_sparse_prefill_pertoken_varlen(const uint16_t* q, const uint16_t* kv_cache, const float* kv_row_scale,
                                       int num_slots,
                                       const int32_t* topk, int64_t ld, int T, int H, int cols, int R,
                                       const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                                       const int32_t* q_pos_start, const int32_t* block_table,
                                       int64_t bt_ld, int page_size, int d_qk, int d_v, float scale,
                                       int32_t* topk_ws, uint16_t* out, float* lse, void* stream);

/* A batch over a paged FP8 cache (kv_scale indexed by cache row when
 * scale_per_row is 1): decodes the pages each request can reach (positions
 * below kv_lens[r], pages 0 .. ceil(kv_lens[r] / page_size) - 1 of its block
 * table row) into ws_cache, request after request -- request r's pages start
 * at compact page off(r) = the reachable pages of requests 0 .. r - 1 --
 * writes each decoded row's scale to ws_row_scale, and writes ws_block_table
 * [R, bt_ld] over ws_cache: off(r) + p for a reachable page p whose page id is
 * valid (0 <= id < num_slots / page_size) and fits the workspace, -1 elsewhere.
 * The batch entry points above then run on (ws_cache, ws_row_scale, ws_pages *
 * page_size rows, ws_block_table) with the same cu_seqlens_q / kv_lens /
 * q_pos_start.  Pages shared by several requests are decoded once per request.
 *   ws_pages      workspace capacity in pages; it must hold the sum over
 *                 requests of ceil(kv_lens[r] / page_size), or the pages past
 *                 it map nowhere (their positions are not selected)
 *   ws_cache      bf16 [ws_pages * page_size, d] (decoded codes, exact)
 *   ws_row_scale  float32 [ws_pages * page_size] (rows of pages that map
 *                 nowhere are not written)
 *   ws_block_table int32 [R, bt_ld]
 * num_slots must be a multiple of page_size; d = 576 or 512.  One kernel is
 * enqueued. */
int dsa_decode_paged_fp8(const uint8_t* cache8, const float* kv_scale, int scale_per_row, int num_slots,
                         int d, int R, const int32_t* kv_lens, const int32_t* block_table, int64_t bt_ld,
                         int page_size, int ws_pages, uint16_t* ws_cache, float* ws_row_scale,
                         int32_t* ws_block_table, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_PREFILL_H */
