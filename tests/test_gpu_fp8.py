"""GPU parity of the FP8 latent entry points against the CPU oracle, through the C ABI.

The oracle's FP8 attention is the per-token definition on the exact element values
e4m3 * scale (float64); nothing below takes a reference value from the GPU.

* the decode pass: every bf16 output bit-identical to the oracle's decode of the codes
  (every E4M3 value is a bf16 number);
* attention over an FP8 latent (grouped and per-token, H 16 / 32 / 128, 576 and 512 wide,
  per-row and single scales) against the oracle;
* the exact fallbacks with row scales: one late key per affected token scores far above
  the rest (the sorted walk's two-pass routine, the 128-row exact kernel);
* the per-token paths past the sorted walk: rows wider than its list (register-ring walk)
  and a cache past 65536 rows (windows of the sorted list);
* a batch over a paged FP8 cache: the compact workspace, its row scales and block table
  exactly, then both batch routings against the oracle on the original paged codes.
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


def decoded_bits(codes):
    """bf16 bit patterns of the exact E4M3 values (oracle decode; exact in float32 and bf16)."""
    v = oracle.fp8_e4m3_to_f64(codes).astype(np.float32)
    bits = v.view(np.uint32)
    assert np.all((bits & 0xFFFF)[~np.isnan(v)] == 0)      # bf16 numbers
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("d", [576, 512])
def test_decode_bit_exact(d):
    from mla_prefill_amd import _lib
    rng = np.random.default_rng(80 + d)
    S = 333
    codes = rng.integers(0, 256, (S, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x5A            # a cache holds no NaN codes
    codes[0, :256] = np.arange(256, dtype=np.uint8)  # every code once
    codes[0, 0x7F] = codes[0, 0xFF] = 0
    out = torch.empty((S, d), dtype=torch.bfloat16, device="cuda")
    _lib.dsa_decode_latent_fp8(dev_u8(codes), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), decoded_bits(codes))


FP8_CASES = [
    # (label, seed, T, S, H, k, cols, P0, d, per_row, mode)
    ("h16_d576_row", 81, 150, 400, 16, 120, 128, 250, 576, True, "locality"),
    ("h16_d512_tensor", 82, 97, 97, 16, 64, 70, 0, 512, False, "uniform"),
    ("h32_d576_tensor", 83, 61, 190, 32, 70, 75, 129, 576, False, "locality"),
    ("h64_d512_row", 86, 37, 160, 64, 90, 90, 123, 512, True, "uniform"),
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


@pytest.mark.parametrize("H,d", [(16, 576), (16, 512), (128, 576)])
def test_fp8_score_jump(H, d):
    """One late key per affected token scores far above the rest (codes +-2 matching head 0's
    query signs, row scale 1 against ~1/100 elsewhere: ~80 base-2 units above the reference),
    so the exact fallbacks run with row scales."""
    from mla_prefill_amd import routings
    rng = np.random.default_rng(87 + H + d)
    T, S, P0 = 24, 200, 176
    q = normal_bf16(rng, (T, H, d))
    codes, scale = normal_fp8(rng, S, d, per_row=True)
    topk = topk_uniform(rng, T, S, 120, 128, P0)
    for t in range(0, T, 3):
        r = t
        codes[r] = np.where(q[t, 0] & 0x8000, 0xC0, 0x40).astype(np.uint8)   # e4m3 -2 / +2
        scale[r] = 1.0
        topk[t][topk[t] == r] = -1
        topk[t, 120] = r
    sc = 1.0 / 16.0
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_fp8(q, codes, scale, topk, S, P0, sc)
    qd, c8, s8, tk = dev_bf16(q), dev_u8(codes), dev_f32(scale), dev_i32(topk)
    out, lse = routings.pertoken_fp8(qd, c8, s8, tk, P0, sc)
    check_attention(out, lse, ref_out, ref_lse, f"fp8 score jump H={H} d={d} per-token")
    out, lse, _ = routings.grouped_fp8(qd, c8, s8, tk, P0, sc)
    check_attention(out, lse, ref_out, ref_lse, f"fp8 score jump H={H} d={d} grouped")


def test_fp8_pertoken_far_positions_and_wide_rows():
    """Per-token over FP8 latents past the sorted walk's simple case: a 70000-row latent
    (two windows of the sorted list) and rows with up to 3000 valid entries (the
    register-ring walk inside the sorted kernel)."""
    from mla_prefill_amd import routings
    rng = np.random.default_rng(88)
    H = 16
    for T, S, k, cols, P0 in ((12, 70000, 300, 320, 70000 - 12), (10, 4000, 3000, 3100, 4000 - 10)):
        q = normal_bf16(rng, (T, H, 576))
        codes, scale = normal_fp8(rng, S, 576, per_row=True)
        topk = topk_uniform(rng, T, S, k, cols, P0)
        ref_out, ref_lse = oracle.pertoken_sparse_mqa_fp8(q, codes, scale, topk, S, P0, 0.0625)
        out, lse = routings.pertoken_fp8(dev_bf16(q), dev_u8(codes), dev_f32(scale), dev_i32(topk), P0, 0.0625)
        check_attention(out, lse, ref_out, ref_lse, f"fp8 per-token S={S} cols={cols}")


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
    ws_cache, ws_scale, wb = routings.decode_paged_fp8(dev_u8(codes), dev_f32(scale), b, ws_pages)
    torch.cuda.synchronize()
    # the compact workspace: request after request, its reachable pages decoded exactly, with
    # the source rows' scales, and the block table over it
    bt = c.block_table
    wbt = wb[3].cpu().numpy()
    ws = ws_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    wsc = ws_scale.cpu().numpy()
    off = 0
    for r, n in enumerate(reach):
        for p in range(bt.shape[1]):
            if p < n:
                assert wbt[r, p] == off + p
                src = bt[r, p] * c.page_size
                dst = (off + p) * c.page_size
                np.testing.assert_array_equal(ws[dst:dst + c.page_size], decoded_bits(codes[src:src + c.page_size]))
                np.testing.assert_array_equal(wsc[dst:dst + c.page_size], scale[src:src + c.page_size])
            else:
                assert wbt[r, p] == -1
        off += n
    # both batch routings over the workspace against the oracle on the original paged codes
    sc = 1.0 / 16.0
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_varlen_fp8(c.q, codes, scale, c.topk, c.cu_seqlens, c.kv_lens,
                                                             c.q_pos_start, c.block_table, c.page_size, sc)
    q, tk = dev_bf16(c.q), dev_i32(c.topk)
    out, lse, _ = routings.grouped_varlen(q, ws_cache, tk, wb, sc, max_groups=c.max_groups(), kv_row_scale=ws_scale)
    check_attention(out, lse, ref_out, ref_lse, f"paged fp8 H={H} grouped")
    out, lse, _ = routings.pertoken_varlen(q, ws_cache, tk, wb, sc, kv_row_scale=ws_scale)
    check_attention(out, lse, ref_out, ref_lse, f"paged fp8 H={H} per-token")
