"""The three routings of DSA sparse prefill, with torch-allocated outputs.

Allocation and argument marshalling only: every step runs in the HIP kernels
of libdsa_prefill.so through the C ABI (``mla_prefill_amd._lib``).
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class UnionBuffers:
    union_idx: torch.Tensor   # int32 [NG, union_pad]
    union_len: torch.Tensor   # int32 [NG]
    mask: torch.Tensor        # uint8 [NG, union_pad]


def alloc_union(T: int, G: int, cols: int, device="cuda") -> UnionBuffers:
    NG = -(-T // G)
    pad = _lib.dsa_union_pad(G, cols)
    return UnionBuffers(torch.empty((NG, pad), dtype=torch.int32, device=device),
                        torch.empty((NG,), dtype=torch.int32, device=device),
                        torch.empty((NG, pad), dtype=torch.uint8, device=device))


def alloc_out(T: int, H: int, dv: int, device="cuda"):
    return (torch.empty((T, H, dv), dtype=torch.bfloat16, device=device),
            torch.empty((T, H), dtype=torch.float32, device=device))


def build_group_union(topk, S: int, q_pos_offset: int, G: int, bufs: UnionBuffers | None = None,
                      stream=None) -> UnionBuffers:
    T, cols = topk.shape
    bufs = bufs or alloc_union(T, G, cols, topk.device)
    _lib.dsa_build_group_union(topk, S, q_pos_offset, G, bufs.union_idx, bufs.union_len, bufs.mask,
                               stream=stream)
    return bufs


def grouped(q, kv, topk, q_pos_offset: int, scale: float, bufs: UnionBuffers | None = None,
            out=None, lse=None, stream=None):
    """Union/mask build followed by grouped attention (G = 128 / H)."""
    T, H, _ = q.shape
    G = 128 // H
    bufs = build_group_union(topk, kv.shape[0], q_pos_offset, G, bufs, stream)
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_grouped(q, kv, bufs.union_idx, bufs.union_len, bufs.mask, scale, out, lse,
                                    stream=stream)
    return out, lse, bufs


def auto(q, kv, topk, q_pos_offset: int, scale: float, bufs: UnionBuffers | None = None, route=None,
         out=None, lse=None, stream=None):
    """Union build, then grouped or per-token attention as chosen on the device from the
    union's size; route[0] == 1 afterwards when the per-token form ran."""
    T, H, _ = q.shape
    bufs = bufs or alloc_union(T, 128 // H, topk.shape[1], q.device)
    if route is None:
        route = torch.zeros(4, dtype=torch.int32, device=q.device)
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_auto(q, kv, topk, q_pos_offset, scale, bufs.union_idx, bufs.union_len, bufs.mask,
                                 route, out, lse, stream=stream)
    return out, lse, bufs, route


def pertoken(q, kv, topk, q_pos_offset: int, scale: float, out=None, lse=None, stream=None):
    T, H, _ = q.shape
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_pertoken(q, kv, topk, q_pos_offset, scale, out, lse, stream=stream)
    return out, lse


def masked_mha(q, k_nope, k_pe, v, topk, q_pos_offset: int, scale: float, mask_ws=None, out=None,
               lse=None, stream=None):
    T, H, _ = q.shape
    S = k_nope.shape[0]
    if mask_ws is None:
        mask_ws = torch.empty((T, (S + 31) // 32), dtype=torch.int32, device=q.device)
    if out is None:
        out, lse = alloc_out(T, H, v.shape[2], q.device)
    _lib.dsa_masked_mha_prefill(q, k_nope, k_pe, v, topk, q_pos_offset, scale, mask_ws, out, lse,
                                stream=stream)
    return out, lse, mask_ws


def dense_mha(q, k_nope, k_pe, v, q_pos_offset: int, scale: float, out=None, lse=None, stream=None):
    T, H, _ = q.shape
    if out is None:
        out, lse = alloc_out(T, H, v.shape[2], q.device)
    _lib.dsa_dense_mha_prefill(q, k_nope, k_pe, v, q_pos_offset, scale, out, lse, stream=stream)
    return out, lse


# ---------------------------------------------------------------------------
# FP8 latent (kv8 uint8 OCP E4M3 codes, kv_scale float32 per row or single)
# ---------------------------------------------------------------------------

def alloc_latent_ws(S: int, d: int, device="cuda"):
    """bf16 workspace for a decoded latent."""
    return torch.empty((S, d), dtype=torch.bfloat16, device=device)


def grouped_fp8(q, kv8, kv_scale, topk, q_pos_offset: int, scale: float, bufs: UnionBuffers | None = None,
                kv_ws=None, out=None, lse=None, stream=None):
    T, H, _ = q.shape
    G = 128 // H
    bufs = build_group_union(topk, kv8.shape[0], q_pos_offset, G, bufs, stream)
    if kv_ws is None:
        kv_ws = alloc_latent_ws(*kv8.shape, q.device)
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_grouped_fp8(q, kv8, kv_scale, bufs.union_idx, bufs.union_len, bufs.mask, scale,
                                        kv_ws, out, lse, stream=stream)
    return out, lse, bufs


def pertoken_fp8(q, kv8, kv_scale, topk, q_pos_offset: int, scale: float, kv_ws=None, out=None, lse=None,
                 stream=None):
    T, H, _ = q.shape
    if kv_ws is None:
        kv_ws = alloc_latent_ws(*kv8.shape, q.device)
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_pertoken_fp8(q, kv8, kv_scale, topk, q_pos_offset, scale, kv_ws, out, lse,
                                         stream=stream)
    return out, lse


def decode_paged_fp8(cache8, kv_scale, batch, ws_pages: int, stream=None):
    """(ws_cache, ws_row_scale, batch over it): the batch's reachable pages decoded to bf16
    (exactly), each workspace row's scale, and the same batch with the block table over the
    workspace."""
    cu, kv_lens, q_pos_start, block_table, page_size = batch
    ws_cache = torch.empty((ws_pages * page_size, cache8.shape[1]), dtype=torch.bfloat16, device=cache8.device)
    ws_scale = torch.empty((ws_pages * page_size,), dtype=torch.float32, device=cache8.device)
    ws_bt = torch.empty_like(block_table)
    _lib.dsa_decode_paged_fp8(cache8, kv_scale, batch, ws_cache, ws_scale, ws_bt, stream=stream)
    return ws_cache, ws_scale, (cu, kv_lens, q_pos_start, ws_bt, page_size)


# ---------------------------------------------------------------------------
# batches of requests over a paged KV cache; `batch` = (cu_seqlens_q, kv_lens,
# q_pos_start, block_table, page_size), int32 device tensors and an int
# ---------------------------------------------------------------------------

@dataclass
class VarlenUnionBuffers:
    group_info: torch.Tensor  # int32 [max_groups, 2]
    union_idx: torch.Tensor   # int32 [max_groups, union_pad]
    union_len: torch.Tensor   # int32 [max_groups]
    mask: torch.Tensor        # uint8 [max_groups, union_pad]


def alloc_union_varlen(max_groups: int, G: int, cols: int, device="cuda") -> VarlenUnionBuffers:
    pad = _lib.dsa_union_pad(G, cols)
    return VarlenUnionBuffers(torch.empty((max_groups, 2), dtype=torch.int32, device=device),
                              torch.empty((max_groups, pad), dtype=torch.int32, device=device),
                              torch.empty((max_groups,), dtype=torch.int32, device=device),
                              torch.empty((max_groups, pad), dtype=torch.uint8, device=device))


def build_group_union_varlen(topk, batch, num_slots: int, G: int, max_groups: int | None = None,
                             bufs: VarlenUnionBuffers | None = None, stream=None) -> VarlenUnionBuffers:
    T, cols = topk.shape
    if bufs is None:
        mg = max_groups if max_groups is not None else _lib.dsa_varlen_group_bound(T, batch[1].shape[0], G)
        bufs = alloc_union_varlen(mg, G, cols, topk.device)
    _lib.dsa_build_group_union_varlen(topk, batch, num_slots, G, bufs.group_info, bufs.union_idx,
                                      bufs.union_len, bufs.mask, stream=stream)
    return bufs


def grouped_varlen(q, kv_cache, topk, batch, scale: float, max_groups: int | None = None,
                   bufs: VarlenUnionBuffers | None = None, out=None, lse=None, kv_row_scale=None, stream=None):
    """Union/mask build of a batch followed by its grouped attention (G = 128 / H); kv_row_scale:
    the cache rows' scales (a decoded FP8 cache) or None."""
    T, H, _ = q.shape
    G = 128 // H
    bufs = build_group_union_varlen(topk, batch, kv_cache.shape[0], G, max_groups, bufs, stream)
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_grouped_varlen(q, kv_cache, bufs.group_info, bufs.union_idx, bufs.union_len,
                                           bufs.mask, scale, out, lse, kv_row_scale=kv_row_scale, stream=stream)
    return out, lse, bufs


def pertoken_varlen(q, kv_cache, topk, batch, scale: float, topk_ws=None, out=None, lse=None, kv_row_scale=None,
                    stream=None):
    T, H, _ = q.shape
    if topk_ws is None:
        topk_ws = torch.empty(topk.shape, dtype=torch.int32, device=q.device)
    if out is None:
        out, lse = alloc_out(T, H, 512, q.device)
    _lib.dsa_sparse_prefill_pertoken_varlen(q, kv_cache, topk, batch, scale, topk_ws, out, lse,
                                            kv_row_scale=kv_row_scale, stream=stream)
    return out, lse, topk_ws
