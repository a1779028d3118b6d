"""GPU parity of the FP8 latent entry points against the CPU oracle, through the C ABI.

* the conversion pass: every bf16 output bit-identical to the oracle's rounding of
  e4m3 * scale (per-row and single scales, both latent widths);
* attention over an FP8 latent (grouped and per-token, H 16 / 32 / 128, 576 and 512
  wide) against the oracle (the latent dequantized to bf16, then the per-token
  definition);
* a batch over a paged FP8 cache: the compact workspace and its block table exactly,
  then both batch routings on it.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_varlen_case, normal_fp8
from synth.gen import normal_bf16, shuffle_rows, topk_locality, topk_uniform
from tests.gpu_helpers import check_attention, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(np.atleast_1d(x), dtype=np.float32)).cuda()


@pytest.mark.parametrize("d", [576, 512])
@pytest.mark.parametrize("per_row", [True, False])
def test_dequant_bit_exact(d, per_row):
    from mla_prefill_amd import _lib
    rng = np.random.default_rng(80 + d + per_row)
    S = 333
    codes = rng.integers(0, 256, (S, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x5A            # a cache holds no NaN codes
    scale = rng.uniform(1e-3, 4.0, S if per_row else 1).astype(np.float32)
    out = torch.empty((S, d), dtype=torch.bfloat16, device="cuda")
    _lib.dsa_dequant_latent_fp8(dev_u8(codes), dev_f32(scale), out)
    torch.cuda.synchronize()
    ref = oracle.dequant_latent_fp8_bf16(codes, scale if per_row else scale[0])
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref)


FP8_CASES = [
    # (label, seed, T, S, H, k, cols, P0, d, per_row, mode)
    ("h16_d576_row", 81, 150, 400, 16, 120, 128, 250, 576, True, "locality"),
    ("h16_d512_tensor", 82, 97, 97, 16, 64, 70, 0, 512, False, "uniform"),
    ("h32_d576_tensor", 83, 61, 190, 32, 70, 75, 129, 576, False, "locality"),
    ("h128_d576_row", 84, 19, 300, 128, 100, 110, 281, 576, True, "locality"),
    ("h128_d512_row", 85, 23, 260, 128, 90, 96, 237, 512, True, "uniform"),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_attention_parity(case):
    from mla_prefill_amd import routings
    label, seed, T, S, H, k, cols, P0, d, per_row, mode = case
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (T, H, d))
    codes, scale = normal_fp8(rng, S, d, per_row)
    topk = (topk_uniform(rng, T, S, k, cols, P0) if mode == "uniform"
            else topk_locality(rng, T, S, k, cols, 128 // H, P0))
    topk = shuffle_rows(topk, seed)
    sc = 1.0 / 16.0
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_fp8(q, codes, scale if per_row else scale[0], topk, S, P0, sc)
    qd, c8, s8, tk = dev_bf16(q), dev_u8(codes), dev_f32(scale), dev_i32(topk)
    out, lse = routings.pertoken_fp8(qd, c8, s8, tk, P0, sc)
    check_attention(out, lse, ref_out, ref_lse, f"{label} per-token fp8")
    out, lse, _ = routings.grouped_fp8(qd, c8, s8, tk, P0, sc)
    check_attention(out, lse, ref_out, ref_lse, f"{label} grouped fp8")


@pytest.mark.parametrize("H", [16, 128])
def test_paged_fp8_batch(H):
    from mla_prefill_amd import routings
    c = make_varlen_case(90 + H, [9, 25, 0, 6], [30, 0, 12, 70], H=H, k=24, cols=28, page_size=8,
                         G=128 // H, mode="locality", values=True)
    rng = np.random.default_rng(91 + H)
    codes, scale = normal_fp8(rng, c.num_slots, 576, per_row=True)
    b = (dev_i32(c.cu_seqlens), dev_i32(c.kv_lens), dev_i32(c.q_pos_start), dev_i32(c.block_table), c.page_size)
    reach = [-(-int(n) // c.page_size) for n in c.kv_lens]
    ws_pages = sum(reach) + 2
    ws_cache, wb = routings.dequant_paged_fp8(dev_u8(codes), dev_f32(scale), b, ws_pages)
    torch.cuda.synchronize()
    # the compact workspace: request after request, its reachable pages, bit-exact
    bt = c.block_table
    wbt = wb[3].cpu().numpy()
    ws = ws_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    conv = oracle.dequant_latent_fp8_bf16(codes, scale)
    off = 0
    for r, n in enumerate(reach):
        for p in range(bt.shape[1]):
            if p < n:
                assert wbt[r, p] == off + p
                src = bt[r, p] * c.page_size
                dst = (off + p) * c.page_size
                np.testing.assert_array_equal(ws[dst:dst + c.page_size], conv[src:src + c.page_size])
            else:
                assert wbt[r, p] == -1
        off += n
    # both batch routings over the workspace against the oracle on the converted cache
    kv_bits = np.zeros((ws_pages * c.page_size, 576), np.uint16)
    kv_bits[:] = ws
    args = (c.cu_seqlens, c.kv_lens, c.q_pos_start, wbt, c.page_size)
    sc = 1.0 / 16.0
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_varlen(c.q, kv_bits, c.topk, *args, sc)
    q, tk = dev_bf16(c.q), dev_i32(c.topk)
    out, lse, _ = routings.grouped_varlen(q, ws_cache, tk, wb, sc, max_groups=c.max_groups())
    check_attention(out, lse, ref_out, ref_lse, f"paged fp8 H={H} grouped")
    out, lse, _ = routings.pertoken_varlen(q, ws_cache, tk, wb, sc)
    check_attention(out, lse, ref_out, ref_lse, f"paged fp8 H={H} per-token")
