"""Shared helpers of the GPU parity tests: device transfer and the parity bar.

Parity bar (the tolerances the method's north star states, plus a per-row bound):
  * union list, union length and membership mask: bit-identical;
  * out: ||out - ref||_F / ||ref||_F <= 3e-3 over the compared tokens, and every
    (token, head) row on its own within ROW_RTOL (a handful of wrong rows cannot
    hide inside the whole-tensor norm);
  * LSE: max |lse - ref| <= 2e-3 over finite entries; -inf entries must match
    exactly, and their out rows must be exactly zero.

Why ROW_RTOL = 1e-2: one row's error comes from the bf16 rounding of the output
(about 2^-9 / sqrt(3) relative per element) and of the probabilities; when one key
dominates a row, the rounding of its probability moves the whole row by up to 2^-9,
so a correct row stays below about 3e-3 relative, while a wrong key set or a wrong
row is off by order 1.
"""

import numpy as np
import torch

OUT_RTOL = 3e-3
LSE_ATOL = 2e-3
ROW_RTOL = 1e-2


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def row_rel_err(o: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative error of every row (last axis) of o against ref; rows whose reference is
    zero are measured against the typical row norm instead."""
    diff = np.linalg.norm(o - ref, axis=-1)
    rn = np.linalg.norm(ref, axis=-1)
    typical = float(np.sqrt(np.mean(rn ** 2))) if rn.size else 1.0
    return diff / np.where(rn > 0, rn, max(typical, 1e-30))


def check_attention(out, lse, ref_out, ref_lse, label=""):
    """out/lse: device tensors restricted to the compared tokens; ref: oracle fp64."""
    o = host_f64(out)
    lv = lse.float().cpu().numpy().astype(np.float64)
    assert o.shape == ref_out.shape, (o.shape, ref_out.shape)
    assert np.all(np.isfinite(o)), f"{label}: non-finite out"
    ref_inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lv), ref_inf), f"{label}: -inf LSE pattern differs"
    assert not np.any(np.isnan(lv)) and not np.any(np.isposinf(lv)), f"{label}: NaN/+inf LSE"
    if ref_inf.any():
        assert np.all(o[ref_inf] == 0.0), f"{label}: empty rows must be exactly zero"
    fin = ~ref_inf
    denom = np.linalg.norm(ref_out)
    rel = np.linalg.norm(o - ref_out) / denom if denom > 0 else np.linalg.norm(o)
    lse_err = float(np.max(np.abs(lv[fin] - ref_lse[fin]))) if fin.any() else 0.0
    rows = row_rel_err(o[fin], ref_out[fin])
    row_max = float(rows.max()) if rows.size else 0.0
    assert rel <= OUT_RTOL, f"{label}: out rel err {rel:.3e} > {OUT_RTOL}"
    assert lse_err <= LSE_ATOL, f"{label}: lse abs err {lse_err:.3e} > {LSE_ATOL}"
    if row_max > ROW_RTOL:
        bad = np.argwhere(row_rel_err(o, ref_out) > ROW_RTOL)[:5].tolist()
        raise AssertionError(f"{label}: worst (token, head) row rel err {row_max:.3e} > {ROW_RTOL} "
                             f"(first offending [token, head] indices {bad})")
    return rel, lse_err


def check_rows_equal(a: torch.Tensor, b: torch.Tensor, label=""):
    """Two GPU results [T, H, d] of the same definition: whole-tensor and per-(token, head)
    relative difference within the parity bars (computed on the device)."""
    a, b = a.float(), b.float()
    rel = (torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b)).item()
    assert rel <= OUT_RTOL, f"{label}: rel diff {rel:.3e}"
    rn = torch.linalg.vector_norm(b, dim=-1)
    typical = torch.sqrt(torch.mean(rn * rn)).clamp_min(1e-30)
    rows = torch.linalg.vector_norm(a - b, dim=-1) / torch.where(rn > 0, rn, typical)
    worst = rows.max().item()
    assert worst <= ROW_RTOL, (f"{label}: worst (token, head) row rel diff {worst:.3e} at "
                               f"{divmod(int(rows.argmax().item()), rows.shape[1])}")
    return rel, worst


def check_union_rows(union_idx, mask, ref_idx, ref_len, ref_mask, label=""):
    """The union buffers against the oracle's: union_len equal, and each row's slots up to the
    next multiple of 64 past its union (the written part) bit-exact; the rest of the row is
    not written by the builder and not compared."""
    ui = union_idx.cpu().numpy() if hasattr(union_idx, "cpu") else np.asarray(union_idx)
    mk = mask.cpu().numpy() if hasattr(mask, "cpu") else np.asarray(mask)
    ref_idx, ref_mask, ref_len = np.asarray(ref_idx), np.asarray(ref_mask), np.asarray(ref_len)
    assert ui.shape == ref_idx.shape and mk.shape == ref_mask.shape, label
    for g in range(ui.shape[0]):
        end = min(ui.shape[1], (int(ref_len[g]) + 63) // 64 * 64)
        np.testing.assert_array_equal(ui[g, :end], ref_idx[g, :end], err_msg=f"{label} union_idx row {g}")
        np.testing.assert_array_equal(mk[g, :end], ref_mask[g, :end], err_msg=f"{label} mask row {g}")
