"""The entry point that allocates nothing (dsa_masked_mha_prefill_noalloc), through the C ABI.

Its output must equal dsa_masked_mha_prefill's (the same kernels over the same bit mask,
kept in the library's static device scratch instead of a caller workspace) bit for bit,
on two calls in a row, the second with a smaller input, and calls past the scratch's
capacity are rejected before anything is enqueued.
"""

import numpy as np
import pytest
import torch

from synth.gen import normal_bf16, topk_locality
from tests.gpu_helpers import dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def _case(seed, T, S, H, k, cols, P0, dn, dr, dv):
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (T, H, dn + dr))
    kn = normal_bf16(rng, (S, H, dn))
    kp = normal_bf16(rng, (S, dr)) if dr else None
    v = normal_bf16(rng, (S, H, dv))
    topk = topk_locality(rng, T, S, k, cols, 8, P0)
    return (dev_bf16(q), dev_bf16(kn), None if kp is None else dev_bf16(kp), dev_bf16(v), dev_i32(topk), P0)


def test_noalloc_equals_workspace_form_twice():
    from mla_prefill_amd import _lib, routings
    cases = [
        # (seed, T, S, H, k, cols, P0, dn, dr, dv): the second call is smaller than the first
        (120, 700, 1500, 4, 200, 210, 800, 256, 0, 256),
        (121, 97, 150, 2, 60, 64, 53, 192, 64, 256),
    ]
    for c in cases:
        print(f"noalloc case {c}", flush=True)
        q, kn, kp, v, tk, P0 = _case(*c)
        T, H = q.shape[0], q.shape[1]
        dv = v.shape[2]
        ref_out, ref_lse, _ = routings.masked_mha(q, kn, kp, v, tk, P0, 0.0625)
        out, lse = routings.alloc_out(T, H, dv)
        out.fill_(7.0)
        lse.fill_(7.0)
        _lib.dsa_masked_mha_prefill_noalloc(q, kn, kp, v, tk, P0, 0.0625, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), c
        assert torch.equal(lse, ref_lse), c


def test_noalloc_rejects_work_past_the_scratch():
    from mla_prefill_amd import _lib
    T, S, H = 16384, 32800, 1
    q = torch.empty((T, H, 256), dtype=torch.bfloat16, device="cuda")
    kn = torch.empty((S, H, 256), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((S, H, 256), dtype=torch.bfloat16, device="cuda")
    tk = torch.full((T, 4), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.DsaError) as err:
        _lib.dsa_masked_mha_prefill_noalloc(q, kn, None, v, tk, 0, 0.0625, out, lse)
    assert err.value.status == -6
