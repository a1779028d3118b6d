"""GPU parity of the batch entry points (requests over a paged KV cache) against
the CPU oracle, through the C ABI.

Batches mix request lengths that are and are not multiples of the group, empty
requests, chunked contexts, shuffled physical pages and page sizes from 4 to 64
rows; the index conversion, group table, union list and mask must be
bit-identical, the attention within the parity bar.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_varlen_case
from synth.gen import shuffle_rows
from tests.gpu_helpers import check_attention, check_union_rows, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from mla_prefill_amd import routings
    return routings


CASES = [
    # (label, seed, q_lens, ctx_lens, H, k, cols, page_size, mode)
    ("mixed_h16", 50, [7, 19, 1, 12], [0, 30, 5, 17], 16, 20, 24, 16, "locality"),
    ("ragged_h32", 51, [9, 3, 14, 8, 1], [11, 0, 6, 40, 2], 32, 16, 16, 4, "uniform"),
    ("h128_g1", 52, [5, 6], [100, 3], 128, 32, 40, 8, "locality"),
    ("long_ctx_h16", 53, [64, 40], [3000, 1500], 16, 512, 520, 64, "locality"),
    ("empty_requests_h64", 54, [0, 10, 0, 5], [5, 0, 7, 20], 64, 12, 14, 8, "uniform"),
]


def device_batch(c):
    return (dev_i32(c.cu_seqlens), dev_i32(c.kv_lens), dev_i32(c.q_pos_start), dev_i32(c.block_table),
            c.page_size)


def oracle_args(c):
    return (c.cu_seqlens, c.kv_lens, c.q_pos_start, c.block_table, c.page_size)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_parity(R, case):
    label, seed, q_lens, ctx_lens, H, k, cols, page, mode = case
    c = make_varlen_case(seed, q_lens, ctx_lens, H=H, k=k, cols=cols, page_size=page, G=128 // H,
                         mode=mode)
    c.topk = shuffle_rows(c.topk, seed)
    G = 128 // H
    print(f"[{label}] T={c.T} R={len(q_lens)} slots={c.num_slots}", flush=True)
    q, kv, tk, b = dev_bf16(c.q), dev_bf16(c.kv_cache), dev_i32(c.topk), device_batch(c)
    scale = 1.0 / 16.0

    # index conversion: bit-exact
    from mla_prefill_amd import _lib
    g = torch.empty_like(tk)
    _lib.dsa_convert_req_index_to_global(tk, b, c.num_slots, g)
    ref_g = oracle.convert_req_index_to_global(c.topk, *oracle_args(c), c.num_slots)
    np.testing.assert_array_equal(g.cpu().numpy(), ref_g)

    # union / mask / group table: bit-exact (two spare groups stay empty)
    mg = c.max_groups() + 2
    out_g, lse_g, bufs = R.grouped_varlen(q, kv, tk, b, scale, max_groups=mg)
    info, ui, ul, mk = oracle.group_union_mask_varlen(c.topk, *oracle_args(c), c.num_slots, G, mg,
                                                      pad=bufs.union_idx.shape[1])
    np.testing.assert_array_equal(bufs.group_info.cpu().numpy(), info)
    np.testing.assert_array_equal(bufs.union_len.cpu().numpy(), ul)
    check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk)

    # attention: both routings against the per-token oracle
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *oracle_args(c), scale)
    check_attention(out_g, lse_g, ref_out, ref_lse, f"{label} grouped")
    out_p, lse_p, _ = R.pertoken_varlen(q, kv, tk, b, scale)
    check_attention(out_p, lse_p, ref_out, ref_lse, f"{label} per-token")


def test_varlen_large_cache_and_score_jump(R):
    """A cache beyond 65536 rows (per-token: the register-ring kernel) and scores that jump
    far above a row's first ones (grouped: the exact fallback path), with both scales."""
    c = make_varlen_case(55, [21, 9], [40, 17], H=16, k=24, cols=24, page_size=1024, spare_pages=70,
                         G=8)
    assert c.num_slots > 65536
    # keys that follow the sign of query dim 0 of the token sharing their index: big jumps
    kvv = c.kv_cache.copy()
    kvv[:, 0] = np.where(np.arange(kvv.shape[0]) % 3 == 0, 0xC000, 0x4000)
    qq = c.q.copy()
    qq[:, :, 0] = 0x4200
    q, kv, tk, b = dev_bf16(qq), dev_bf16(kvv), dev_i32(c.topk), device_batch(c)
    for scale in (0.7, -0.7):
        ref_out, ref_lse = oracle.pertoken_sparse_mqa_varlen(qq, kvv, c.topk, *oracle_args(c), scale)
        out_g, lse_g, _ = R.grouped_varlen(q, kv, tk, b, scale)
        check_attention(out_g, lse_g, ref_out, ref_lse, f"grouped jump, scale {scale}")
        out_p, lse_p, _ = R.pertoken_varlen(q, kv, tk, b, scale)
        check_attention(out_p, lse_p, ref_out, ref_lse, f"per-token jump, scale {scale}")


def test_varlen_single_request_matches_single_sequence(R):
    """One request with an identity page table: the batch entry points reproduce the
    single-sequence ones bit for bit."""
    c = make_varlen_case(56, [45], [70], H=16, k=40, cols=48, page_size=5, spare_pages=0, G=8)
    c.block_table[0] = np.arange(c.block_table.shape[1])
    q, kv, tk, b = dev_bf16(c.q), dev_bf16(c.kv_cache), dev_i32(c.topk), device_batch(c)
    S, P0 = int(c.kv_lens[0]), int(c.q_pos_start[0])
    o1, l1, _ = R.grouped_varlen(q, kv[:S].contiguous(), tk, b, 0.1)
    o2, l2, _ = R.grouped(q, kv[:S].contiguous(), tk, P0, 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("H", [16, 128])
def test_varlen_latent512(R, H):
    """A batch over a paged cache of 512-wide latent rows (no rope part): both routings."""
    c = make_varlen_case(56 + H, [11, 30, 4], [40, 0, 90], H=H, k=24, cols=28, page_size=8, G=128 // H,
                         mode="locality", d_qk=512)
    q, kv, tk, b = dev_bf16(c.q), dev_bf16(c.kv_cache), dev_i32(c.topk), device_batch(c)
    scale = 1.0 / 16.0
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *oracle_args(c), scale)
    out_g, lse_g, _ = R.grouped_varlen(q, kv, tk, b, scale, max_groups=c.max_groups())
    check_attention(out_g, lse_g, ref_out, ref_lse, f"d512 H={H} grouped batch")
    out_p, lse_p, _ = R.pertoken_varlen(q, kv, tk, b, scale)
    check_attention(out_p, lse_p, ref_out, ref_lse, f"d512 H={H} per-token batch")
