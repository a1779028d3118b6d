"""ctypes binding of libdsa_prefill.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch
tensors that live on the GPU; it passes their data pointers, sizes and the
current HIP stream to the library and raises ``DsaError`` on a non-zero status.
Every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing, importing this module fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_prefill.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python -m mla_prefill_amd.build` "
        "(hipcc --offload-arch=gfx950); there is no non-HIP fallback")

lib = ctypes.CDLL(_LIB_PATH)

_i32, _i64, _f32, _vp, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "dsa_abi_version": ([], _i32),
    "dsa_status_string": ([_i32], ctypes.c_char_p),
    "dsa_union_pad": ([_i32, _i32], _i32),
    "dsa_masked_mha_workspace_bytes": ([_i32, _i32], _sz),
    "dsa_select_routing": ([_i32, _i32, _i64, _i32, _i32, _i32], _i32),
    "dsa_build_group_union": ([_vp, _i64, _i32, _i32, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp], _i32),
    "dsa_sparse_prefill_grouped": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                    _vp, _vp, _vp], _i32),
    "dsa_sparse_prefill_pertoken": ([_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32,
                                     _vp, _vp, _vp], _i32),
    "dsa_sparse_prefill_auto": ([_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32, _i32,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "dsa_masked_mha_prefill": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _i64, _f32, _vp, _vp, _vp, _vp], _i32),
    "dsa_masked_mha_prefill_noalloc": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _i64, _f32, _vp, _vp, _vp], _i32),
    "dsa_dense_mha_prefill": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                               _vp, _vp, _vp], _i32),
    "dsa_decode_latent_fp8": ([_vp, _i32, _i32, _vp, _vp], _i32),
    "dsa_sparse_prefill_grouped_fp8": ([_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _f32, _vp, _vp, _vp, _vp], _i32),
    "dsa_sparse_prefill_pertoken_fp8": ([_vp, _vp, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _i32,
                                         _f32, _vp, _vp, _vp, _vp], _i32),
    "dsa_decode_paged_fp8": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp],
                             _i32),
    "dsa_varlen_group_bound": ([_i32, _i32, _i32], _i32),
    "dsa_convert_req_index_to_global": ([_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                         _vp, _vp], _i32),
    "dsa_build_group_union_varlen": ([_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                      _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
    "dsa_sparse_prefill_grouped_varlen": ([_vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                           _i32, _i32, _f32, _vp, _vp, _vp], _i32),
    "dsa_sparse_prefill_pertoken_varlen": ([_vp, _vp, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                                            _vp, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp],
                                           _i32),
}
for _name, (_args, _ret) in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

EXPORTED = tuple(_SIGNATURES)


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({lib.dsa_status_string(status).decode()})")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DsaError(fn, status)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.numel() and not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if t.numel() and not t.is_contiguous() and t.dim() > 1 and t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _bits(t):
    """bf16 tensors travel as their 16-bit patterns."""
    if t is None:
        return None
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected bf16 bits, got {t.dtype}")
    return t


def _topk_ld(topk):
    if topk.dtype != torch.int32:
        raise TypeError("topk must be int32")
    if topk.dim() != 2 or topk.stride(1) != 1:
        raise ValueError("topk must be [T, ld] with unit column stride")
    return topk.stride(0) if topk.shape[0] > 1 else max(topk.shape[1], 1)


def dsa_abi_version() -> int:
    return lib.dsa_abi_version()


def dsa_status_string(status: int) -> str:
    return lib.dsa_status_string(status).decode()


def dsa_union_pad(G: int, cols: int) -> int:
    v = lib.dsa_union_pad(G, cols)
    _check("dsa_union_pad", v if v < 0 else 0)
    return v


def dsa_masked_mha_workspace_bytes(T: int, S: int) -> int:
    return lib.dsa_masked_mha_workspace_bytes(T, S)


ROUTING_NAMES = {1: "dense", 2: "masked", 3: "grouped", 4: "per-token"}


def dsa_select_routing(T: int, S: int, q_pos_offset: int, H: int, k: int, mha_dv: int) -> str:
    """Name of the routing the library picks for one chunk ("dense", "masked", "grouped" or
    "per-token"); mha_dv is the value width of the caller's MHA geometry (256 or 128), or 0
    when it cannot run the MHA forms."""
    r = lib.dsa_select_routing(T, S, q_pos_offset, H, k, int(mha_dv))
    _check("dsa_select_routing", min(r, 0))
    return ROUTING_NAMES[r]


def dsa_build_group_union(topk, S, q_pos_offset, G, union_idx, union_len, head_group_mask,
                          cols=None, stream=None):
    T = topk.shape[0]
    cols = topk.shape[1] if cols is None else cols
    _check("dsa_build_group_union", lib.dsa_build_group_union(
        _ptr(topk), _topk_ld(topk), T, cols, S, q_pos_offset, G, union_idx.shape[1],
        _ptr(union_idx), _ptr(union_len), _ptr(head_group_mask), _stream(stream)))


def dsa_sparse_prefill_grouped(q, kv, union_idx, union_len, head_group_mask, scale, out, lse,
                               stream=None):
    T, H, d_qk = q.shape
    S = kv.shape[0]
    _check("dsa_sparse_prefill_grouped", lib.dsa_sparse_prefill_grouped(
        _ptr(_bits(q)), _ptr(_bits(kv)), _ptr(union_idx), _ptr(union_len), _ptr(head_group_mask),
        T, H, S, union_idx.shape[1], d_qk, out.shape[2], scale, _ptr(_bits(out)), _ptr(lse),
        _stream(stream)))


def dsa_sparse_prefill_pertoken(q, kv, topk, q_pos_offset, scale, out, lse, cols=None, stream=None):
    T, H, d_qk = q.shape
    S = kv.shape[0]
    cols = topk.shape[1] if cols is None else cols
    _check("dsa_sparse_prefill_pertoken", lib.dsa_sparse_prefill_pertoken(
        _ptr(_bits(q)), _ptr(_bits(kv)), _ptr(topk), _topk_ld(topk), T, H, S, cols, q_pos_offset,
        d_qk, out.shape[2], scale, _ptr(_bits(out)), _ptr(lse), _stream(stream)))


def dsa_sparse_prefill_auto(q, kv, topk, q_pos_offset, scale, union_idx, union_len, head_group_mask, route, out,
                            lse, cols=None, stream=None):
    T, H, d_qk = q.shape
    S = kv.shape[0]
    cols = topk.shape[1] if cols is None else cols
    _check("dsa_sparse_prefill_auto", lib.dsa_sparse_prefill_auto(
        _ptr(_bits(q)), _ptr(_bits(kv)), _ptr(topk), _topk_ld(topk), T, H, S, cols, q_pos_offset, d_qk,
        out.shape[2], scale, union_idx.shape[1], _ptr(union_idx), _ptr(union_len), _ptr(head_group_mask),
        _ptr(route), _ptr(_bits(out)), _ptr(lse), _stream(stream)))


def dsa_masked_mha_prefill(q, k_nope, k_pe, v, topk, q_pos_offset, scale, mask_ws, out, lse,
                           cols=None, stream=None):
    T, H, dqk = q.shape
    S, _, dn = k_nope.shape
    dr = 0 if k_pe is None else k_pe.shape[-1]
    dv = v.shape[2]
    cols = topk.shape[1] if cols is None else cols
    _check("dsa_masked_mha_prefill", lib.dsa_masked_mha_prefill(
        _ptr(_bits(q)), _ptr(_bits(k_nope)), _ptr(_bits(k_pe)), _ptr(_bits(v)), _ptr(topk),
        _topk_ld(topk), T, S, H, dn, dr, dv, cols, q_pos_offset, scale, _ptr(mask_ws),
        _ptr(_bits(out)), _ptr(lse), _stream(stream)))


def dsa_masked_mha_prefill_noalloc(q, k_nope, k_pe, v, topk, q_pos_offset, scale, out, lse, cols=None,
                                   stream=None):
    """dsa_masked_mha_prefill with the mask in the library's static scratch (no workspace)."""
    T, H, dqk = q.shape
    S, _, dn = k_nope.shape
    dr = 0 if k_pe is None else k_pe.shape[-1]
    dv = v.shape[2]
    cols = topk.shape[1] if cols is None else cols
    _check("dsa_masked_mha_prefill_noalloc", lib.dsa_masked_mha_prefill_noalloc(
        _ptr(_bits(q)), _ptr(_bits(k_nope)), _ptr(_bits(k_pe)), _ptr(_bits(v)), _ptr(topk),
        _topk_ld(topk), T, S, H, dn, dr, dv, cols, q_pos_offset, scale, _ptr(_bits(out)), _ptr(lse),
        _stream(stream)))


def dsa_dense_mha_prefill(q, k_nope, k_pe, v, q_pos_offset, scale, out, lse, stream=None):
    T, H, dqk = q.shape
    S, _, dn = k_nope.shape
    dr = 0 if k_pe is None else k_pe.shape[-1]
    dv = v.shape[2]
    _check("dsa_dense_mha_prefill", lib.dsa_dense_mha_prefill(
        _ptr(_bits(q)), _ptr(_bits(k_nope)), _ptr(_bits(k_pe)), _ptr(_bits(v)), T, S, H, dn, dr, dv,
        q_pos_offset, scale, _ptr(_bits(out)), _ptr(lse), _stream(stream)))


# ---------------------------------------------------------------------------
# FP8 latent: kv8 uint8 [S, d] OCP E4M3 codes, kv_scale float32 [S] (per row) or [1]
# ---------------------------------------------------------------------------

def _fp8(kv8, kv_scale):
    if kv8.dtype != torch.uint8:
        raise TypeError("FP8 codes travel as uint8")
    if kv_scale.dtype != torch.float32:
        raise TypeError("kv_scale must be float32")
    per_row = int(kv_scale.numel() != 1)
    if per_row and kv_scale.numel() < kv8.shape[0]:
        raise ValueError("kv_scale needs one value per row (or a single value)")
    return per_row


def dsa_decode_latent_fp8(kv8, out, stream=None):
    if kv8.dtype != torch.uint8:
        raise TypeError("FP8 codes travel as uint8")
    S, d = kv8.shape
    _check("dsa_decode_latent_fp8", lib.dsa_decode_latent_fp8(_ptr(kv8), S, d, _ptr(_bits(out)), _stream(stream)))


def dsa_sparse_prefill_grouped_fp8(q, kv8, kv_scale, union_idx, union_len, head_group_mask, scale, kv_ws,
                                   out, lse, stream=None):
    T, H, d_qk = q.shape
    S = kv8.shape[0]
    _check("dsa_sparse_prefill_grouped_fp8", lib.dsa_sparse_prefill_grouped_fp8(
        _ptr(_bits(q)), _ptr(kv8), _ptr(kv_scale), _fp8(kv8, kv_scale), _ptr(union_idx), _ptr(union_len),
        _ptr(head_group_mask), T, H, S, union_idx.shape[1], d_qk, out.shape[2], scale, _ptr(_bits(kv_ws)),
        _ptr(_bits(out)), _ptr(lse), _stream(stream)))


def dsa_sparse_prefill_pertoken_fp8(q, kv8, kv_scale, topk, q_pos_offset, scale, kv_ws, out, lse, cols=None,
                                    stream=None):
    T, H, d_qk = q.shape
    S = kv8.shape[0]
    cols = topk.shape[1] if cols is None else cols
    _check("dsa_sparse_prefill_pertoken_fp8", lib.dsa_sparse_prefill_pertoken_fp8(
        _ptr(_bits(q)), _ptr(kv8), _ptr(kv_scale), _fp8(kv8, kv_scale), _ptr(topk), _topk_ld(topk), T, H, S,
        cols, q_pos_offset, d_qk, out.shape[2], scale, _ptr(_bits(kv_ws)), _ptr(_bits(out)), _ptr(lse),
        _stream(stream)))


# ---------------------------------------------------------------------------
# batches of requests over a paged KV cache.  A batch is passed as the tuple
# (cu_seqlens_q, kv_lens, q_pos_start, block_table, page_size) of int32 device
# tensors (block_table [R, bt_ld]) and the page size.
# ---------------------------------------------------------------------------

def _batch(batch):
    cu, kv_lens, q_pos_start, block_table, page_size = batch
    for t in (cu, kv_lens, q_pos_start, block_table):
        if t.dtype != torch.int32:
            raise TypeError("batch tensors must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [R, bt_ld] with unit column stride")
    R = kv_lens.shape[0]
    bt_ld = block_table.stride(0) if block_table.shape[0] > 1 else block_table.shape[1]
    return R, _ptr(cu), _ptr(kv_lens), _ptr(q_pos_start), _ptr(block_table), bt_ld, page_size


def dsa_varlen_group_bound(T: int, R: int, G: int) -> int:
    v = lib.dsa_varlen_group_bound(T, R, G)
    _check("dsa_varlen_group_bound", v if v < 0 else 0)
    return v


def dsa_convert_req_index_to_global(topk, batch, num_slots, topk_global, cols=None, stream=None):
    T = topk.shape[0]
    cols = topk.shape[1] if cols is None else cols
    R, cu, kl, qs, bt, bt_ld, ps = _batch(batch)
    _check("dsa_convert_req_index_to_global", lib.dsa_convert_req_index_to_global(
        _ptr(topk), _topk_ld(topk), T, cols, R, cu, kl, qs, bt, bt_ld, ps, num_slots, _ptr(topk_global),
        _stream(stream)))


def dsa_build_group_union_varlen(topk, batch, num_slots, G, group_info, union_idx, union_len,
                                 head_group_mask, cols=None, stream=None):
    T = topk.shape[0]
    cols = topk.shape[1] if cols is None else cols
    R, cu, kl, qs, bt, bt_ld, ps = _batch(batch)
    _check("dsa_build_group_union_varlen", lib.dsa_build_group_union_varlen(
        _ptr(topk), _topk_ld(topk), T, cols, R, cu, kl, qs, bt, bt_ld, ps, num_slots, G,
        group_info.shape[0], union_idx.shape[1], _ptr(group_info), _ptr(union_idx), _ptr(union_len),
        _ptr(head_group_mask), _stream(stream)))


def _row_scale(kv_cache, kv_row_scale):
    if kv_row_scale is None:
        return None
    if kv_row_scale.dtype != torch.float32 or kv_row_scale.numel() < kv_cache.shape[0]:
        raise ValueError("kv_row_scale must be float32 with one value per cache row")
    return _ptr(kv_row_scale)


def dsa_sparse_prefill_grouped_varlen(q, kv_cache, group_info, union_idx, union_len, head_group_mask,
                                      scale, out, lse, kv_row_scale=None, stream=None):
    T, H, d_qk = q.shape
    _check("dsa_sparse_prefill_grouped_varlen", lib.dsa_sparse_prefill_grouped_varlen(
        _ptr(_bits(q)), _ptr(_bits(kv_cache)), _row_scale(kv_cache, kv_row_scale), kv_cache.shape[0],
        _ptr(group_info), group_info.shape[0],
        _ptr(union_idx), _ptr(union_len), _ptr(head_group_mask), T, H, union_idx.shape[1], d_qk,
        out.shape[2], scale, _ptr(_bits(out)), _ptr(lse), _stream(stream)))


def dsa_sparse_prefill_pertoken_varlen(q, kv_cache, topk, batch, scale, topk_ws, out, lse, cols=None,
                                       kv_row_scale=None, stream=None):
    T, H, d_qk = q.shape
    cols = topk.shape[1] if cols is None else cols
    R, cu, kl, qs, bt, bt_ld, ps = _batch(batch)
    _check("dsa_sparse_prefill_pertoken_varlen", lib.dsa_sparse_prefill_pertoken_varlen(
        _ptr(_bits(q)), _ptr(_bits(kv_cache)), _row_scale(kv_cache, kv_row_scale), kv_cache.shape[0], _ptr(topk), _topk_ld(topk), T, H, cols, R,
        cu, kl, qs, bt, bt_ld, ps, d_qk, out.shape[2], scale, _ptr(topk_ws), _ptr(_bits(out)), _ptr(lse),
        _stream(stream)))


def dsa_decode_paged_fp8(cache8, kv_scale, batch, ws_cache, ws_row_scale, ws_block_table, stream=None):
    """Decode the pages a batch can reach into ws_cache [ws_pages * page_size, d], their rows'
    scales into ws_row_scale, and write ws_block_table [R, bt_ld] over the workspace."""
    _, kv_lens, _, block_table, page_size = batch
    b = _batch(batch)
    R, bt_ld = b[0], b[5]
    num_slots, d = cache8.shape
    if ws_block_table.dtype != torch.int32 or ws_block_table.shape != block_table.shape:
        raise ValueError("ws_block_table must be int32 shaped like block_table")
    ws_pages = ws_cache.shape[0] // page_size
    if ws_row_scale.dtype != torch.float32 or ws_row_scale.numel() < ws_pages * page_size:
        raise ValueError("ws_row_scale must be float32 with one value per workspace row")
    _check("dsa_decode_paged_fp8", lib.dsa_decode_paged_fp8(
        _ptr(cache8), _ptr(kv_scale), _fp8(cache8, kv_scale), num_slots, d, R, _ptr(kv_lens), _ptr(block_table),
        bt_ld, page_size, ws_pages, _ptr(_bits(ws_cache)), _ptr(ws_row_scale), _ptr(ws_block_table),
        _stream(stream)))
