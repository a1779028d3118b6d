"""Shared helpers of the GPU parity tests: device transfer and the parity bar.

Parity bar (the tolerances the method's north star states):
  * union list, union length and membership mask: bit-identical;
  * out: ||out - ref||_F / ||ref||_F <= 3e-3 over the compared tokens;
  * LSE: max |lse - ref| <= 2e-3 over finite entries; -inf entries must match
    exactly, and their out rows must be exactly zero.
"""

import numpy as np
import torch

OUT_RTOL = 3e-3
LSE_ATOL = 2e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


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
    assert rel <= OUT_RTOL, f"{label}: out rel err {rel:.3e} > {OUT_RTOL}"
    assert lse_err <= LSE_ATOL, f"{label}: lse abs err {lse_err:.3e} > {LSE_ATOL}"
    return rel, lse_err
