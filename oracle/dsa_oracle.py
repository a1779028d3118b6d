"""CPU oracle (numpy, float64) for DSA sparse-MLA prefill attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path (no kernels, headers, helpers or tables) and the HIP path
never calls it.

Every function is the plain definition of what the pages compute, written out
slowly and obviously; none of the kernels' blocking, tiling, online softmax or
bitmap tricks appear here.  Pages cited:

* [MASKED] "[2/N][Attention] Enable masked MHA for sparse MLA prefills"
  (vllm-project/vllm PR #48770) -- Purpose section: below a length threshold a
  masked MHA simulates DSA (mask = causal AND top-k membership); for chunks no
  longer than the top-k every causal key is selected and a plain causal MHA
  (the dense shortcut) gives the same result.
* [NOPE] "[Perf][GLM-5.3-Flash] Dense/masked-MHA sparse prefill for the NoPE
  (256, 0, 256) layout + skip the NoPE K concat" (vllm-project/vllm PR #55738)
  -- commit messages (K is k_nope itself when the rope part is empty; K is
  k_nope concatenated with the broadcast k_pe otherwise) and the Purpose
  section (per-token top-k MQA kernel over the latent).
* [GROUPED] "[Perf][DSA] Grouped sparse prefill with the FlashMLA
  head-group-mask kernel" (JaredforReal/vllm PR #6) -- commit message and the
  "How" section: 128 // num_heads consecutive tokens form 128 pseudo-heads over
  the sorted union of their top-k rows; a per-token membership mask restricts
  each token's heads to its own top-k, which reproduces per-token sparse
  attention exactly; the union is padded to a multiple of a block; the GLM
  comment on that page: -1 entries pad a wider (2176-column) top-k buffer.

Readings where the pages are silent (each also listed in the design notes):

* Selection: sel(t) = {x in topk[t, :cols] : 0 <= x < S and x <= q_pos_offset + t}.
  -1 padding, out-of-range and non-causal entries are ignored in every routing.
  Entries of a row are distinct (an indexer top-k is a set); the oracle raises
  on duplicates.
* Softmax scale multiplies the raw dot products; LSE is the natural log of the
  sum of exp(scaled logits).  An empty selection gives out = 0 and LSE = -inf.
* Values: V is the first d_v (= 512) dims of the latent row.
* Grouping: group g holds tokens gG .. min(T, gG + G) - 1 with G = 128 / H;
  pseudo-head r = i * H + h for token gG + i and head h.
* Union list: strictly ascending, -1 padded to union_pad = ceil(G*cols/64)*64.
* head_group_mask: uint8 [NG, union_pad]; bit i of slot j is set iff token
  gG + i selects union position j; padding slots are 0.
* FP8 KV latent (the pages only gate quantized caches off the grouped path and
  define no format): OCP E4M3 codes (uint8) with a float32 scale per row or one
  for the whole cache; element (x, i) = e4m3(kv8[x, i]) * scale, exactly (in
  float64).  Attention over such a cache is the per-token definition on those
  exact values (scores and values both use the scaled elements).
* Batches of requests over a paged KV cache ([GROUPED] "How": groups are
  consecutive tokens of one request, and the union's request-local positions
  become physical KV rows through the request's index conversion before the
  attention): request r owns query tokens cu[r] .. cu[r+1] - 1; its token i sits
  at position q_pos_start[r] + i; it may select positions 0 <= x < kv_len[r]
  (and x <= its position); position x lives in physical row
  block_table[r][x // page_size] * page_size + x % page_size of the cache.
  Positions whose row falls outside the cache are ignored.  Groups are numbered
  request by request (ceil(n_r / G) per request) and never cross a request.

Pins: see ``tests/test_oracle_pins.py`` (library routines, closed forms,
brute-force set arithmetic, invariants).  No function here is parity-unpinned.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

UNION_BLOCK = 64


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def union_pad(G: int, cols: int) -> int:
    """Padded length of one group's union list: ceil(G * cols / 64) * 64."""
    return -(-(G * cols) // UNION_BLOCK) * UNION_BLOCK


def selected_positions(row: np.ndarray, S: int, pos: int) -> np.ndarray:
    """sel(t) for one top-k row, in row order (see the module docstring)."""
    row = np.asarray(row, dtype=np.int64)
    sel = row[(row >= 0) & (row < S) & (row <= pos)]
    if np.unique(sel).size != sel.size:
        raise ValueError("a top-k row holds the same valid position twice")
    return sel


def softmax_attention(qrows: np.ndarray, keys: np.ndarray, values: np.ndarray,
                      scale: float):
    """Exact softmax attention of query rows over a key set.

    qrows [R, d], keys [n, d], values [n, dv] (float64).
    Returns out [R, dv] = softmax(scale * q k^T) v and lse [R] = log sum exp(scale * q k^T).
    """
    R = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((R, values.shape[1])), np.full(R, -np.inf)
    logits = scale * (qrows @ keys.T)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    total = e.sum(axis=1, keepdims=True)
    out = (e @ values) / total
    lse = m[:, 0] + np.log(total[:, 0])
    return out, lse


def _as_scale(scale: float) -> float:
    # the GPU receives the scale as float32; the oracle uses that same value
    return float(np.float32(scale))


def _tokens(T: int, tokens: Optional[Iterable[int]]) -> np.ndarray:
    return np.arange(T) if tokens is None else np.asarray(list(tokens), dtype=np.int64)


# ---------------------------------------------------------------------------
# per-token sparse MQA  ([NOPE] Purpose; [GROUPED] commit message)
# ---------------------------------------------------------------------------

def pertoken_sparse_mqa(q: np.ndarray, kv: np.ndarray, topk: np.ndarray, S: int,
                        q_pos_offset: int, scale: float, d_v: int = 512,
                        tokens: Optional[Iterable[int]] = None):
    """Every token t attends, for all H heads, over the latent rows sel(t).

    q uint16 [T, H, d_qk], kv uint16 [S, d_qk], topk int32 [T, cols].
    Returns (out float64 [n, H, d_v], lse float64 [n, H]) for the requested tokens.
    """
    T, H, _ = q.shape
    scale = _as_scale(scale)
    toks = _tokens(T, tokens)
    kv64 = bf16_to_f64(kv[:S])
    out = np.zeros((toks.size, H, d_v))
    lse = np.full((toks.size, H), -np.inf)
    for n, t in enumerate(toks):
        sel = selected_positions(topk[t], S, q_pos_offset + int(t))
        keys = kv64[sel]
        out[n], lse[n] = softmax_attention(bf16_to_f64(q[t]), keys, keys[:, :d_v], scale)
    return out, lse


# ---------------------------------------------------------------------------
# union list + head_group_mask  ([GROUPED] commit message, "How" section)
# ---------------------------------------------------------------------------

def group_union_mask(topk: np.ndarray, S: int, q_pos_offset: int, G: int,
                     pad: Optional[int] = None):
    """Sorted union of each group's selections and the per-token membership mask.

    Returns union_idx int32 [NG, pad] (-1 padded), union_len int32 [NG],
    mask uint8 [NG, pad].
    """
    T, cols = topk.shape
    pad = union_pad(G, cols) if pad is None else pad
    NG = -(-T // G)
    union_idx = np.full((NG, pad), -1, dtype=np.int32)
    union_len = np.zeros(NG, dtype=np.int32)
    mask = np.zeros((NG, pad), dtype=np.uint8)
    for g in range(NG):
        members = [selected_positions(topk[t], S, q_pos_offset + t)
                   for t in range(g * G, min(T, g * G + G))]
        U = np.unique(np.concatenate(members)) if members else np.zeros(0, np.int64)
        n = U.size
        union_idx[g, :n] = U
        union_len[g] = n
        for i, sel in enumerate(members):
            mask[g, :n] |= (np.isin(U, sel).astype(np.uint8) << np.uint8(i))
    return union_idx, union_len, mask


# ---------------------------------------------------------------------------
# grouped sparse MQA over the union  ([GROUPED] commit message, "How")
# ---------------------------------------------------------------------------

def grouped_sparse_mqa(q: np.ndarray, kv: np.ndarray, union_idx: np.ndarray,
                       union_len: np.ndarray, mask: np.ndarray, scale: float,
                       d_v: int = 512, groups: Optional[Iterable[int]] = None):
    """Pseudo-head r = i*H + h of group g attends over the union slots j whose
    mask bit i is set.  Returns (out [T, H, d_v], lse [T, H]); tokens of groups
    not requested stay at out 0 / lse -inf.
    """
    T, H, _ = q.shape
    G = 128 // H
    scale = _as_scale(scale)
    S = kv.shape[0]
    kv64 = bf16_to_f64(kv)
    out = np.zeros((T, H, d_v))
    lse = np.full((T, H), -np.inf)
    gs = range(union_len.size) if groups is None else groups
    for g in gs:
        n = int(union_len[g])
        U = union_idx[g, :n].astype(np.int64)
        bits = mask[g, :n]
        if np.any((U < 0) | (U >= S)):
            raise ValueError("union list holds an out-of-range position")
        for i in range(G):
            t = g * G + i
            if t >= T:
                break
            keys = kv64[U[((bits >> i) & 1) == 1]]
            out[t], lse[t] = softmax_attention(bf16_to_f64(q[t]), keys, keys[:, :d_v], scale)
    return out, lse


# ---------------------------------------------------------------------------
# masked dense MHA  ([MASKED] Purpose; [NOPE] commit messages)
# ---------------------------------------------------------------------------

def masked_mha(q: np.ndarray, k_nope: np.ndarray, k_pe: Optional[np.ndarray],
               v: np.ndarray, topk: np.ndarray, S: int, q_pos_offset: int, scale: float,
               tokens: Optional[Iterable[int]] = None):
    """Dense MHA over all S keys with mask = causal AND top-k membership.

    q uint16 [T, H, dn + dr]; k_nope [S, H, dn]; k_pe [S, dr] or None (dr = 0:
    K is k_nope itself); v [S, H, dv].  Masked logits are -inf, so a token
    with no allowed key gets out 0 and LSE -inf.
    """
    T, H, _ = q.shape
    scale = _as_scale(scale)
    toks = _tokens(T, tokens)
    kn = bf16_to_f64(k_nope[:S])
    kp = bf16_to_f64(k_pe[:S]) if k_pe is not None and k_pe.shape[-1] > 0 else None
    vv = bf16_to_f64(v[:S])
    dv = v.shape[2]
    positions = np.arange(S)
    out = np.zeros((toks.size, H, dv))
    lse = np.full((toks.size, H), -np.inf)
    for n, t in enumerate(toks):
        member = np.zeros(S, dtype=bool)
        member[selected_positions(topk[t], S, q_pos_offset + int(t))] = True
        allowed = member & (positions <= q_pos_offset + int(t))
        if not allowed.any():
            continue
        qt = bf16_to_f64(q[t])
        for h in range(H):
            K = kn[:, h, :] if kp is None else np.concatenate([kn[:, h, :], kp], axis=1)
            logits = scale * (K @ qt[h])
            logits[~allowed] = -np.inf
            m = logits.max()
            e = np.exp(logits - m)
            total = e.sum()
            out[n, h] = (e @ vv[:, h, :]) / total
            lse[n, h] = m + math.log(total)
    return out, lse


def dense_causal_mha(q: np.ndarray, k_nope: np.ndarray, k_pe: Optional[np.ndarray],
                     v: np.ndarray, S: int, q_pos_offset: int, scale: float,
                     tokens: Optional[Iterable[int]] = None):
    """Plain causal MHA: token t attends over every key x <= q_pos_offset + t (x < S).

    [MASKED] Purpose: the dense shortcut for chunks no longer than the top-k,
    where every causal key is selected.  Layouts as ``masked_mha``.
    """
    T, H, _ = q.shape
    scale = _as_scale(scale)
    toks = _tokens(T, tokens)
    kn = bf16_to_f64(k_nope[:S])
    kp = bf16_to_f64(k_pe[:S]) if k_pe is not None and k_pe.shape[-1] > 0 else None
    vv = bf16_to_f64(v[:S])
    out = np.zeros((toks.size, H, v.shape[2]))
    lse = np.full((toks.size, H), -np.inf)
    for n, t in enumerate(toks):
        last = min(q_pos_offset + int(t), S - 1)   # keys 0 .. last
        qt = bf16_to_f64(q[t])
        for h in range(H):
            K = kn[: last + 1, h, :]
            if kp is not None:
                K = np.concatenate([K, kp[: last + 1]], axis=1)
            o, l = softmax_attention(qt[h][None], K, vv[: last + 1, h, :], scale)
            out[n, h], lse[n, h] = o[0], l[0]
    return out, lse


# ---------------------------------------------------------------------------
# FP8 KV latent  ([GROUPED] "How": the grouped path is gated off for quantized
# KV caches; the pages give no FP8 format -- see the module docstring)
# ---------------------------------------------------------------------------

def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (uint8): sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 holds the subnormals m * 2^-9; S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def dequant_latent_fp8(kv8: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Latent rows of an FP8 cache: element (x, i) = e4m3(kv8[x, i]) * scale[x] (float64).

    scale: float32 [S] per row, or a single float32 for the whole cache."""
    v = fp8_e4m3_to_f64(kv8)
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return v * (sc.reshape(-1, 1) if sc.ndim == 1 else sc)


def pertoken_sparse_mqa_fp8(q: np.ndarray, kv8: np.ndarray, scale_kv: np.ndarray, topk: np.ndarray,
                            S: int, q_pos_offset: int, scale: float, d_v: int = 512,
                            tokens: Optional[Iterable[int]] = None):
    """Per-token sparse MQA over an FP8 latent: ``pertoken_sparse_mqa``'s definition on the
    exact element values e4m3 * scale (``dequant_latent_fp8``)."""
    T, H, _ = q.shape
    scale = _as_scale(scale)
    toks = _tokens(T, tokens)
    sc = np.asarray(scale_kv, dtype=np.float32)
    kv64 = dequant_latent_fp8(kv8[:S], sc[:S] if sc.ndim else sc)
    out = np.zeros((toks.size, H, d_v))
    lse = np.full((toks.size, H), -np.inf)
    for n, t in enumerate(toks):
        sel = selected_positions(topk[t], S, q_pos_offset + int(t))
        keys = kv64[sel]
        out[n], lse[n] = softmax_attention(bf16_to_f64(q[t]), keys, keys[:, :d_v], scale)
    return out, lse


# ---------------------------------------------------------------------------
# batches of requests over a paged KV cache  ([GROUPED] "How": groups of
# consecutive tokens of a request; union positions mapped to physical rows)
# ---------------------------------------------------------------------------

def request_of_tokens(cu_seqlens: np.ndarray) -> np.ndarray:
    """Request index of every query token (cu_seqlens [R + 1], ascending)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    owner = np.zeros(int(cu[-1]), dtype=np.int64)
    for r in range(cu.size - 1):
        owner[cu[r]:cu[r + 1]] = r
    return owner


def physical_row(block_table: np.ndarray, r: int, x: int, page_size: int) -> int:
    """Cache row of request r's position x."""
    return int(block_table[r, x // page_size]) * page_size + x % page_size


def token_position(cu_seqlens, q_pos_start, r: int, t: int) -> int:
    return int(q_pos_start[r]) + (t - int(cu_seqlens[r]))


def selected_local_positions(topk_row, kv_len: int, pos: int, block_table, r: int,
                             page_size: int, num_slots: int) -> np.ndarray:
    """Request-local positions a token selects whose physical row is in the cache."""
    sel = selected_positions(topk_row, kv_len, pos)
    keep = [x for x in sel if 0 <= physical_row(block_table, r, int(x), page_size) < num_slots]
    return np.asarray(keep, dtype=np.int64)


def convert_req_index_to_global(topk, cu_seqlens, kv_lens, q_pos_start, block_table,
                                page_size: int, num_slots: int) -> np.ndarray:
    """Each top-k entry as a physical cache row, -1 where it selects nothing.

    topk int32 [T, cols] of request-local positions; returns int32 [T, cols].
    """
    T, cols = topk.shape
    owner = request_of_tokens(cu_seqlens)
    out = np.full((T, cols), -1, dtype=np.int32)
    for t in range(T):
        r = int(owner[t])
        pos = token_position(cu_seqlens, q_pos_start, r, t)
        for c in range(cols):
            x = int(topk[t, c])
            if 0 <= x < int(kv_lens[r]) and x <= pos:
                row = physical_row(block_table, r, x, page_size)
                if 0 <= row < num_slots:
                    out[t, c] = row
    return out


def pertoken_sparse_mqa_varlen(q, kv_cache, topk, cu_seqlens, kv_lens, q_pos_start, block_table,
                               page_size: int, scale: float, d_v: int = 512,
                               tokens: Optional[Iterable[int]] = None):
    """Per-token sparse MQA of a batch of requests over a paged cache [num_slots, d_qk]
    (bf16 bit patterns)."""
    return _pertoken_varlen(q, lambda rows: bf16_to_f64(kv_cache[rows]), kv_cache.shape[0], topk, cu_seqlens,
                            kv_lens, q_pos_start, block_table, page_size, scale, d_v, tokens)


def pertoken_sparse_mqa_varlen_fp8(q, cache8, scale_kv, topk, cu_seqlens, kv_lens, q_pos_start, block_table,
                                   page_size: int, scale: float, d_v: int = 512,
                                   tokens: Optional[Iterable[int]] = None):
    """Per-token sparse MQA of a batch over a paged FP8 cache (codes [num_slots, d_qk], scale
    per cache row or one for the cache): the exact element values e4m3 * scale."""
    sc = np.asarray(scale_kv, dtype=np.float32)

    def rows_of(rows):
        return dequant_latent_fp8(cache8[rows], sc[rows] if sc.ndim else sc)

    return _pertoken_varlen(q, rows_of, cache8.shape[0], topk, cu_seqlens, kv_lens, q_pos_start, block_table,
                            page_size, scale, d_v, tokens)


def _pertoken_varlen(q, rows_of, num_slots, topk, cu_seqlens, kv_lens, q_pos_start, block_table,
                     page_size: int, scale: float, d_v: int, tokens):
    T, H, _ = q.shape
    scale = _as_scale(scale)
    owner = request_of_tokens(cu_seqlens)
    toks = _tokens(T, tokens)
    out = np.zeros((toks.size, H, d_v))
    lse = np.full((toks.size, H), -np.inf)
    for n, t in enumerate(toks):
        r = int(owner[t])
        pos = token_position(cu_seqlens, q_pos_start, r, int(t))
        xs = selected_local_positions(topk[t], int(kv_lens[r]), pos, block_table, r, page_size,
                                      num_slots)
        rows = [physical_row(block_table, r, int(x), page_size) for x in xs]
        keys = rows_of(np.asarray(rows, dtype=np.int64)) if rows else np.zeros((0, q.shape[2]))
        out[n], lse[n] = softmax_attention(bf16_to_f64(q[t]), keys, keys[:, :d_v], scale)
    return out, lse


def varlen_groups(cu_seqlens, G: int):
    """(first token, token count) of every group, request by request."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    groups = []
    for r in range(cu.size - 1):
        for t0 in range(int(cu[r]), int(cu[r + 1]), G):
            groups.append((t0, min(G, int(cu[r + 1]) - t0)))
    return groups


def group_union_mask_varlen(topk, cu_seqlens, kv_lens, q_pos_start, block_table, page_size: int,
                            num_slots: int, G: int, max_groups: int, pad: Optional[int] = None):
    """Union (as physical rows, ascending in request-local position) and membership mask of
    every group of a batch.

    Returns group_info int32 [max_groups, 2] (first token, token count; 0, 0 past the last
    group), union_idx int32 [max_groups, pad], union_len int32 [max_groups],
    mask uint8 [max_groups, pad].
    """
    T, cols = topk.shape
    pad = union_pad(G, cols) if pad is None else pad
    owner = request_of_tokens(cu_seqlens)
    groups = varlen_groups(cu_seqlens, G)
    if len(groups) > max_groups:
        raise ValueError("max_groups is smaller than the batch's group count")
    info = np.zeros((max_groups, 2), dtype=np.int32)
    union_idx = np.full((max_groups, pad), -1, dtype=np.int32)
    union_len = np.zeros(max_groups, dtype=np.int32)
    mask = np.zeros((max_groups, pad), dtype=np.uint8)
    for g, (t0, n) in enumerate(groups):
        info[g] = (t0, n)
        r = int(owner[t0])
        members = [selected_local_positions(topk[t], int(kv_lens[r]),
                                            token_position(cu_seqlens, q_pos_start, r, t),
                                            block_table, r, page_size, num_slots)
                   for t in range(t0, t0 + n)]
        U = np.unique(np.concatenate(members)) if members else np.zeros(0, np.int64)
        k = U.size
        union_idx[g, :k] = [physical_row(block_table, r, int(x), page_size) for x in U]
        union_len[g] = k
        for i, sel in enumerate(members):
            mask[g, :k] |= (np.isin(U, sel).astype(np.uint8) << np.uint8(i))
    return info, union_idx, union_len, mask


def grouped_sparse_mqa_varlen(q, kv_cache, group_info, union_idx, union_len, mask, scale: float,
                              d_v: int = 512, groups: Optional[Iterable[int]] = None):
    """Rows of group g (its tokens x H heads) over the union rows whose mask bit is set."""
    T, H, _ = q.shape
    scale = _as_scale(scale)
    num_slots = kv_cache.shape[0]
    out = np.zeros((T, H, d_v))
    lse = np.full((T, H), -np.inf)
    gs = range(group_info.shape[0]) if groups is None else groups
    for g in gs:
        t0, n = int(group_info[g, 0]), int(group_info[g, 1])
        k = int(union_len[g])
        rows = union_idx[g, :k].astype(np.int64)
        bits = mask[g, :k]
        if np.any((rows < 0) | (rows >= num_slots)):
            raise ValueError("union list holds a row outside the cache")
        for i in range(n):
            keys = bf16_to_f64(kv_cache[rows[((bits >> i) & 1) == 1]])
            out[t0 + i], lse[t0 + i] = softmax_attention(bf16_to_f64(q[t0 + i]), keys, keys[:, :d_v], scale)
    return out, lse
