"""GPU parity of every entry point against the CPU oracle, through the C ABI.

Sizes here finish in seconds on the oracle yet span several kernel tiles and
end on ragged tails (T not a multiple of the group, top-k widths that are not
multiples of the tile, -1 padding shuffled through the rows, chunked context).
Full-size configurations are covered by test_gpu_fullsize.py.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_case
from synth.gen import normal_bf16, shuffle_rows, topk_locality, topk_uniform, widen
from tests.gpu_helpers import check_attention, check_union_rows, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from mla_prefill_amd import routings
    return routings


def small_mqa(seed, T, S, H, k, cols, G, P0, mode="locality", shuffle=False, d=576):
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    if mode == "uniform":
        topk = topk_uniform(rng, T, S, k, cols, P0)
    else:
        topk = topk_locality(rng, T, S, k, cols, G, P0)
    if shuffle:
        topk = shuffle_rows(topk, seed + 1)
    return q, kv, topk


MQA_CASES = [
    # (label, seed, T, S, H, k, cols, P0, mode, shuffle)
    ("h16_ragged", 1, 203, 203, 16, 96, 100, 0, "locality", False),
    ("h16_ctx_shuffled", 2, 150, 420, 16, 130, 137, 270, "locality", True),
    ("h16_uniform", 3, 97, 97, 16, 64, 64, 0, "uniform", False),
    ("h32", 4, 61, 190, 32, 70, 75, 129, "locality", True),
    ("h64", 5, 37, 160, 64, 90, 90, 123, "uniform", False),
    ("h128", 6, 19, 300, 128, 100, 110, 281, "locality", True),
]


@pytest.mark.parametrize("case", MQA_CASES, ids=[c[0] for c in MQA_CASES])
def test_union_bit_exact(R, case):
    label, seed, T, S, H, k, cols, P0, mode, shuffle = case
    G = 128 // H
    _, _, topk = small_mqa(seed, T, S, H, k, cols, G, P0, mode, shuffle)
    bufs = R.build_group_union(dev_i32(topk), S, P0, G)
    ui, ul, mk = oracle.group_union_mask(topk, S, P0, G)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bufs.union_len.cpu().numpy(), ul)
    check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk)


def test_union_dense_and_sparse_segments(R):
    """The builder's compaction: each group mixes a dense run (most positions of a
    1500-wide range selected by some member) with sparse picks far away, entries at the
    window edge (32767, 32768), at the first and the last position a member may select,
    and rows of 16-entry vectors and of odd width; group lengths are not multiples of 16.
    Over 40000 positions (two windows, sparse segments) and 5000 (segments of 2048
    positions: the dense run makes one wave's segment dense, its neighbour's mixed).
    Union, lengths and masks bit-exact."""
    rng = np.random.default_rng(43)
    for cols, G, T, S in ((768, 8, 19, 40000), (771, 4, 9, 40000), (768, 8, 19, 5000)):
        P0 = S - T
        topk = np.full((T, cols), -1, np.int32)
        for t in range(T):
            pos = P0 + t
            base = 1000 + 13 * (t // G)
            dense = base + rng.permutation(1500)[: 500 + 100 * (t % G)]   # members cover the run
            far = rng.choice(np.arange(3000, pos + 1), size=120, replace=False)
            edge = np.array([0, 32767, 32768, pos, pos - 1, 31999, 32000])
            sel = np.unique(np.concatenate([dense, far, edge]))
            sel = sel[sel <= pos][: cols - 3]
            row = np.concatenate([rng.permutation(sel), [S + 5, -3, pos + 1]])   # ignored entries
            topk[t, : len(row)] = row[:cols]
        ui, ul, mk = oracle.group_union_mask(topk, S, P0, G)
        bufs = R.build_group_union(dev_i32(topk), S, P0, G)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bufs.union_len.cpu().numpy(), ul)
        check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk, f"cols {cols} G {G}")


@pytest.mark.parametrize("case", MQA_CASES, ids=[c[0] for c in MQA_CASES])
def test_pertoken_parity(R, case):
    label, seed, T, S, H, k, cols, P0, mode, shuffle = case
    q, kv, topk = small_mqa(seed, T, S, H, k, cols, 128 // H, P0, mode, shuffle)
    scale = 1.0 / 16.0
    out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, scale)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, label)


@pytest.mark.parametrize("case", MQA_CASES, ids=[c[0] for c in MQA_CASES])
def test_grouped_parity(R, case):
    label, seed, T, S, H, k, cols, P0, mode, shuffle = case
    G = 128 // H
    q, kv, topk = small_mqa(seed, T, S, H, k, cols, G, P0, mode, shuffle)
    scale = 1.0 / 16.0
    out, lse, _ = R.grouped(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, scale)
    # grouped must reproduce per-token attention: compare with the per-token oracle
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, label)


def test_tiny_config_all_mqa_routings(R):
    c = make_case(CONFIGS["c1_tiny"])
    cfg = c.cfg
    q, kv, tk = dev_bf16(c.q), dev_bf16(c.kv), dev_i32(c.topk)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(c.q, c.kv, c.topk, cfg.S, 0, cfg.scale)
    o1, l1 = R.pertoken(q, kv, tk, 0, cfg.scale)
    check_attention(o1, l1, ref_out, ref_lse, "c1 per-token")
    o2, l2, bufs = R.grouped(q, kv, tk, 0, cfg.scale)
    check_attention(o2, l2, ref_out, ref_lse, "c1 grouped")
    ui, ul, mk = oracle.group_union_mask(c.topk, cfg.S, 0, cfg.G)
    np.testing.assert_array_equal(bufs.union_len.cpu().numpy(), ul)
    check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk)
    og, lg = oracle.grouped_sparse_mqa(c.q, c.kv, ui, ul, mk, cfg.scale)
    check_attention(o2, l2, og, lg, "c1 grouped vs grouped oracle")


def test_empty_and_degenerate_rows(R):
    rng = np.random.default_rng(9)
    T, S, H = 21, 40, 16
    q = normal_bf16(rng, (T, H, 576))
    kv = normal_bf16(rng, (S, 576))
    topk = np.full((T, 70), -1, np.int32)
    topk[3, 5] = 2                 # a single selected row
    topk[4, :3] = [S + 5, -9, 39]  # nothing valid (39 > position 4)
    topk[7, 10:18] = np.arange(8)  # every causal position of token 7
    for t in range(12, T):
        topk[t, 60:60 + 5] = rng.choice(t + 1, 5, replace=False)
    scale = 0.0625
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, 0, scale)
    qd, kvd, tkd = dev_bf16(q), dev_bf16(kv), dev_i32(topk)
    out, lse = R.pertoken(qd, kvd, tkd, 0, scale)
    check_attention(out, lse, ref_out, ref_lse, "per-token degenerate")
    out, lse, bufs = R.grouped(qd, kvd, tkd, 0, scale)
    check_attention(out, lse, ref_out, ref_lse, "grouped degenerate")
    ui, ul, mk = oracle.group_union_mask(topk, S, 0, 8)
    check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk)


def test_single_token_and_single_group(R):
    rng = np.random.default_rng(10)
    S, H = 300, 16
    for T in (1, 8):
        q = normal_bf16(rng, (T, H, 576))
        kv = normal_bf16(rng, (S, 576))
        topk = topk_uniform(rng, T, S, 200, 256, S - T)
        ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, S - T, 0.1)
        out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), S - T, 0.1)
        check_attention(out, lse, ref_out, ref_lse, f"T={T} per-token")
        out, lse, _ = R.grouped(dev_bf16(q), dev_bf16(kv), dev_i32(topk), S - T, 0.1)
        check_attention(out, lse, ref_out, ref_lse, f"T={T} grouped")


def test_strided_topk_and_wider_buffer(R):
    """topk with a leading dimension larger than the used columns, and -1 widening."""
    q, kv, topk = small_mqa(11, 40, 120, 16, 50, 60, 8, 80)
    wide = widen(topk, 100)
    scale = 0.07
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, 120, 80, scale)
    tk = dev_i32(wide)[:, :60]                      # ld = 100, cols = 60
    out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), tk, 80, scale)
    check_attention(out, lse, ref_out, ref_lse, "strided topk")
    out2, lse2, _ = R.grouped(dev_bf16(q), dev_bf16(kv), dev_i32(wide), 80, scale)
    check_attention(out2, lse2, ref_out, ref_lse, "wider buffer grouped")


def test_deterministic(R):
    q, kv, topk = small_mqa(12, 64, 200, 16, 100, 120, 8, 136)
    qd, kvd, tkd = dev_bf16(q), dev_bf16(kv), dev_i32(topk)
    a = R.pertoken(qd, kvd, tkd, 136, 0.1)
    b = R.pertoken(qd, kvd, tkd, 136, 0.1)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    c = R.grouped(qd, kvd, tkd, 136, 0.1)
    d = R.grouped(qd, kvd, tkd, 136, 0.1)
    assert torch.equal(c[0].view(torch.int16), d[0].view(torch.int16)) and torch.equal(c[1], d[1])


def test_pertoken_far_positions_and_wide_rows(R):
    """Per-token rows with positions beyond 65535 (two windows of the sorted list), and rows
    with up to 3000 valid entries (more than the sorted list holds: the register-ring walk
    inside the sorted kernel)."""
    rng = np.random.default_rng(14)
    H = 16
    for T, S, k, cols, P0 in ((12, 70000, 300, 320, 70000 - 12), (10, 4000, 3000, 3100, 4000 - 10)):
        q = normal_bf16(rng, (T, H, 576))
        kv = normal_bf16(rng, (S, 576))
        topk = topk_uniform(rng, T, S, k, cols, P0)
        ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.0625)
        out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, 0.0625)
        check_attention(out, lse, ref_out, ref_lse, f"per-token S={S} cols={cols}")


def test_pertoken_sorted_windows(R):
    """The sorted walk over a 300000-row latent: three 131072-position sort chunks, five
    65536-row windows of the sorted list, rows at every window edge, a window holding a single
    row (steps that cross several window starts), -1, out-of-range and non-causal entries."""
    rng = np.random.default_rng(31)
    T, S, H, cols = 6, 300000, 16, 300
    P0 = S - T
    q = normal_bf16(rng, (T, H, 576))
    kv = normal_bf16(rng, (S, 576))
    topk = np.full((T, cols), -1, np.int32)
    for t in range(T):
        pos = P0 + t
        sel = {0, 65535, 65536, 131071, 131072, 196607, 196608, 262143, 262144, pos}
        for lo, hi, n in ((1, 65534, 40), (65537, 131070, 3), (131073, 196606, 150), (196609, 262142, 1),
                          (262145, pos - 1, 17)):
            while sum(lo <= x <= hi for x in sel) < n:
                sel.add(int(rng.integers(lo, hi + 1)))
        row = sorted(sel) + [S, S + 7, -5]                       # out of range: ignored
        if t < T - 1:
            row += [int(rng.integers(pos + 1, S))]                 # not causal: ignored
        row = [row[i] for i in rng.permutation(len(row))]
        topk[t, :len(row)] = row
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.0625)
    out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "per-token S=300000 windows")


def test_pertoken_sort_crowded_entries(R):
    """Entries packed into a few bitmap words far from 0: each token's 2048 entries lie among
    the 2100 positions up to its own (positions past 131072, so in the second sort chunk and in
    the third 65536-row window), one token takes every position of a 2048-wide range, and the
    rows arrive in a shuffled order.  The rank of an entry is the set bits below it, so
    nearly full words test the within-word count; the list must come out sorted."""
    rng = np.random.default_rng(37)
    T, H, k, cols = 5, 16, 2048, 2176
    S = 140000
    P0 = S - T
    q = normal_bf16(rng, (T, H, 576))
    kv = normal_bf16(rng, (S, 576))
    topk = np.full((T, cols), -1, np.int32)
    for t in range(T):
        pos = P0 + t
        if t == 0:
            sel = np.arange(pos - k + 1, pos + 1)                   # every position of the range
        else:
            sel = pos - rng.choice(2100, size=k, replace=False)
        topk[t, :k] = rng.permutation(sel)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.0625)
    out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "per-token crowded entries")


AUTO_CASES = [
    # (label, seed, T, S, H, k, P0, mode, the form expected to run: 0 grouped, 1 per-token)
    ("h16_locality", 41, 400, 1200, 16, 256, 800, "locality", 0),
    ("h16_uniform", 42, 400, 2400, 16, 256, 2000, "uniform", 1),
    ("h32_uniform", 43, 240, 3000, 32, 200, 2760, "uniform", 1),
    ("h64_locality", 44, 130, 900, 64, 300, 770, "locality", 0),
    ("h16_short_rows", 45, 70, 70, 16, 64, 0, "uniform", None),  # early tokens: few keys each
]


@pytest.mark.parametrize("case", AUTO_CASES, ids=[c[0] for c in AUTO_CASES])
def test_auto_routing(R, case):
    """The routing chosen on the device from the union's size: the chosen form runs (route
    words), its result matches the oracle, and the union tiles it counted are the union's."""
    label, seed, T, S, H, k, P0, mode, expect = case
    q, kv, topk = small_mqa(seed, T, S, H, k, k, 128 // H, P0, mode, True)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.0625)
    out, lse, bufs, route = R.auto(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, f"auto {label}")
    rt = route.cpu().numpy()
    _, ul, _ = oracle.group_union_mask(topk, S, P0, 128 // H)
    assert rt[2] == int(np.sum((np.asarray(ul) + 31) // 32))
    assert rt[0] + rt[1] == 1
    if expect is not None:
        assert rt[0] == expect, (label, rt)


def test_latent_past_2gib(R):
    """Both routings over a latent of 1.9 M rows (2.19 GB): row offsets past 2^31 bytes, where
    the grouped kernel's copies take full 64-bit addresses.  Only the selected rows hold values
    (the rest stay zero on the device); the oracle runs on those rows alone, renumbered in
    order, which leaves every token's selection and therefore its attention unchanged."""
    rng = np.random.default_rng(35)
    T, S, H, k = 24, 1_900_000, 16, 96
    P0 = S - T
    limit = (1 << 31) // (576 * 2)                                  # first row past 2 GiB
    topk = np.full((T, k + 4), -1, np.int32)
    for t in range(T):
        far = rng.choice(np.arange(limit, P0), 40, replace=False)
        near = rng.choice(np.arange(0, limit), k - 40, replace=False)
        row = np.concatenate([far, near])
        topk[t, :k] = row[rng.permutation(k)]
    rows = np.unique(topk[topk >= 0])
    vals = normal_bf16(rng, (rows.size, 576))
    q = normal_bf16(rng, (T, H, 576))
    kv = torch.zeros((S, 576), dtype=torch.bfloat16, device="cuda")
    kv[torch.from_numpy(rows.astype(np.int64)).cuda()] = dev_bf16(vals)
    topk_c = np.where(topk >= 0, np.searchsorted(rows, topk), -1).astype(np.int32)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, vals, topk_c, rows.size, rows.size, 0.0625)
    qd, tk = dev_bf16(q), dev_i32(topk)
    out, lse, _ = R.grouped(qd, kv, tk, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "grouped, latent past 2 GiB")
    out, lse = R.pertoken(qd, kv, tk, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "per-token, latent past 2 GiB")
    del kv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H", [48, 112])
def test_pertoken_head_counts_without_grouped_form(R, H):
    """Head counts the per-token kernel takes (multiples of 16) but 128 / H is no group size."""
    q, kv, topk = small_mqa(15 + H, 33, 150, H, 60, 64, 1, 117, "uniform", True)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, 150, 117, 0.0625)
    out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), 117, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, f"per-token H={H}")


def test_grouped_chunked_block_order_with_a_ragged_tail(R):
    """Enough groups (100 at H = 16, 157 at H = 32) that the launch maps most blocks to XCD
    chunks and the rest (a partial round of chunks) one to one: every group must be computed
    exactly once.  Every token is compared with the per-token oracle; also the 128-row kernel
    in per-token mode over 150 tokens at H = 128."""
    for seed, T, S, H, k in ((48, 800, 900, 16, 96), (49, 628, 700, 32, 80), (50, 150, 400, 128, 64)):
        q, kv, topk = small_mqa(seed, T, S, H, k, k, max(1, 128 // H), S - T, "locality", True)
        ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, S - T, 0.0625)
        if H < 128:
            out, lse, _ = R.grouped(dev_bf16(q), dev_bf16(kv), dev_i32(topk), S - T, 0.0625)
        else:
            out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), S - T, 0.0625)
        check_attention(out, lse, ref_out, ref_lse, f"T={T} H={H} chunked block order")


def test_pertoken_h128_trailing_slots(R):
    """The 128-row kernel in per-token mode stops at the tile of the row's last valid slot.
    Rows here end in -1 padding, in non-causal or out-of-range entries (not valid either),
    hold their last valid entry past column 2048 (the prologue's second scan), in the very
    last column, in the first tile only, or hold none at all; a 2300-column buffer."""
    rng = np.random.default_rng(47)
    T, S, H, cols = 9, 3000, 128, 2300
    P0 = S - T
    q = normal_bf16(rng, (T, H, 576))
    kv = normal_bf16(rng, (S, 576))
    topk = np.full((T, cols), -1, np.int32)
    for t in range(T):
        pos = P0 + t
        if t == 8:
            continue                                                  # nothing valid
        n = (40, 700, 1500, 2000, 2100, 2299, 5, 300)[t]
        topk[t, :n] = rng.choice(pos + 1, size=n, replace=False)
    topk[0, 40:60] = P0 + 5                                           # non-causal for token 0
    topk[1, 700:720] = S + 3                                          # out of range
    topk[4, 2100:2105] = -7
    unused = lambda t: int(np.setdiff1d(np.arange(P0), topk[t])[0])
    topk[4, 2150] = unused(4)                                         # last valid slot past 2048
    topk[5, cols - 1] = unused(5)                                     # the very last column
    topk[7, 300:] = P0 + 8                                            # non-causal for all of them
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.0625)
    out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "per-token H=128 trailing slots")


def test_grouped_far_positions(R):
    """The union builder's position windows past 65535 (a 70000-row latent, chunk at its end)."""
    q, kv, topk = small_mqa(16, 24, 70000, 16, 300, 320, 8, 70000 - 24, "uniform", True)
    ui, ul, mk = oracle.group_union_mask(topk, 70000, 70000 - 24, 8)
    out, lse, bufs = R.grouped(dev_bf16(q), dev_bf16(kv), dev_i32(topk), 70000 - 24, 0.0625)
    np.testing.assert_array_equal(bufs.union_len.cpu().numpy(), ul)
    check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, 70000, 70000 - 24, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "grouped S=70000")


def test_large_score_jump_and_negative_scale(R):
    """Scores that jump far above everything earlier in the row (one key per affected token
    scores ~900 raw units on head 0, ~80 in base-2 softmax units, placed late in the row),
    and a negative softmax scale on the same inputs."""
    rng = np.random.default_rng(13)
    T, S, H, P0 = 24, 200, 16, 176
    q = normal_bf16(rng, (T, H, 576))
    kv = normal_bf16(rng, (S, 576))
    topk = topk_uniform(rng, T, S, 120, 128, P0)
    for t in range(0, T, 3):
        r = t                                          # a distinct, causally valid row per token
        kv[r] = np.where(q[t, 0] & 0x8000, 0xC000, 0x4000).astype(np.uint16)  # bf16 -2 / +2
        topk[t][topk[t] == r] = -1
        topk[t, 120] = r
    for scale in (0.0625, -0.0625):
        ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale)
        qd, kvd, tkd = dev_bf16(q), dev_bf16(kv), dev_i32(topk)
        out, lse = R.pertoken(qd, kvd, tkd, P0, scale)
        check_attention(out, lse, ref_out, ref_lse, f"per-token score jump, scale {scale}")
        out, lse, _ = R.grouped(qd, kvd, tkd, P0, scale)
        check_attention(out, lse, ref_out, ref_lse, f"grouped score jump, scale {scale}")


def _late_topk(rng, T, G, P0, cols, first_keys, late_from):
    """The first token of every group selects keys 0 .. first_keys - 1 and some late ones; the
    other tokens select only keys at or after late_from (so, sorted, their first selected union
    entry sits first_keys slots in).  Every row keeps 8 slots of -1 padding."""
    topk = np.full((T, cols), -1, np.int32)
    for t in range(T):
        late = rng.choice(np.arange(late_from, P0 + t + 1), cols - first_keys - 8, replace=False)
        sel = np.concatenate([np.arange(first_keys), late]) if t % G == 0 else late
        topk[t, :len(sel)] = rng.permutation(sel)
    return topk


def _add_jumps(q, kv_rows, topk, tokens, keys, head=0, dims=None, mag=(0xC000, 0x4000)):
    """Key row x (one per token, selected by that token alone) set to +-2 (or mag) along the
    token's query on one head: its score lies far above every earlier score of the row."""
    for t, x in zip(tokens, keys):
        for u in range(topk.shape[0]):
            topk[u][topk[u] == x] = -1
        slot = int(np.flatnonzero(topk[t] == -1)[0])
        topk[t, slot] = x
        qrow = q[t, head] if dims is None else q[t, head, :dims]
        kv_rows[x] = np.where(qrow & 0x8000, mag[0], mag[1]).astype(np.uint16)


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("jump", [False, True], ids=["plain", "jump"])
def test_grouped_late_reference(R, H, jump):
    """Rows whose first selected key sits several union tiles in (their token selects nothing
    among the group's first 100 union entries): the grouped kernel takes row maxima until
    every row of a wave has its reference.  With `jump`, a key near the end of the union
    scores far above the references (~330 base-2 units: its probability would overflow) after
    the maxima are no longer taken, which the probability sum catches (the group goes through
    the exact kernel)."""
    rng = np.random.default_rng(17 + H + jump)
    G = 128 // H
    T, S = 2 * G, 700
    P0 = S - T
    q = normal_bf16(rng, (T, H, 576))
    kv = normal_bf16(rng, (S, 576))
    topk = _late_topk(rng, T, G, P0, 160, 100, 300)
    if jump:
        toks = list(range(1, T, 3))
        _add_jumps(q, kv, topk, toks, [650 + i for i in range(len(toks))], mag=(0xC100, 0x4100))  # +-8
    scale = 0.0625
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale)
    qd, kvd, tkd = dev_bf16(q), dev_bf16(kv), dev_i32(topk)
    out, lse, _ = R.grouped(qd, kvd, tkd, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, f"grouped late reference H={H} jump={jump}")
    out, lse = R.pertoken(qd, kvd, tkd, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, f"per-token late reference H={H} jump={jump}")


@pytest.mark.parametrize("jump", [False, True], ids=["plain", "jump"])
def test_masked_mha_late_reference(R, jump):
    """Masked MHA rows whose selected keys all lie past key 200 (their first six 32-key tiles
    hold nothing for them): maxima until every row of a wave has its reference; with `jump`,
    a late key scores far above the reference afterwards (~150 base-2 units: its probability
    would overflow), which the row's sum catches (the tile goes through the exact kernel)."""
    rng = np.random.default_rng(53 + jump)
    T, S, H, P0 = 300, 300, 2, 0
    q = normal_bf16(rng, (T, H, 256))
    kn = normal_bf16(rng, (S, H, 256))
    v = normal_bf16(rng, (S, H, 256))
    topk = np.full((T, 70), -1, np.int32)
    for t in range(T):
        lo = 200 if t >= 260 else 0
        sel = rng.choice(np.arange(lo, t + 1), min(60, t + 1 - lo), replace=False)
        topk[t, :len(sel)] = sel
    if jump:
        toks = [270, 281, 299]
        _add_jumps(q, kn[:, 0], topk, toks, [262, 275, 290], mag=(0xC100, 0x4100))  # +-8
    out, lse, _ = R.masked_mha(dev_bf16(q), dev_bf16(kn), None, dev_bf16(v), dev_i32(topk), P0, 0.0625)
    ref_out, ref_lse = oracle.masked_mha(q, kn, None, v, topk, S, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, f"masked late reference jump={jump}")


# ---------------------------------------------------------------------------
# the 512-wide latent (no rope part: K = V = the whole row)
# ---------------------------------------------------------------------------

D512_CASES = [c for c in MQA_CASES if c[0] != "h16_uniform"]


@pytest.mark.parametrize("case", D512_CASES, ids=[c[0] for c in D512_CASES])
def test_latent512_parity(R, case):
    label, seed, T, S, H, k, cols, P0, mode, shuffle = case
    G = 128 // H
    q, kv, topk = small_mqa(seed + 40, T, S, H, k, cols, G, P0, mode, shuffle, d=512)
    scale = 1.0 / 16.0
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale)
    qd, kvd, tkd = dev_bf16(q), dev_bf16(kv), dev_i32(topk)
    out, lse = R.pertoken(qd, kvd, tkd, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, f"{label} d512 per-token")
    out, lse, _ = R.grouped(qd, kvd, tkd, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, f"{label} d512 grouped")


def test_latent512_far_positions_and_wide_rows(R):
    """The register-ring per-token kernel at 512 dims (positions past 65535, rows wider than
    the sorted walk takes)."""
    rng = np.random.default_rng(44)
    H = 16
    for T, S, k, cols, P0 in ((12, 70000, 300, 320, 70000 - 12), (10, 4000, 3000, 3100, 4000 - 10)):
        q = normal_bf16(rng, (T, H, 512))
        kv = normal_bf16(rng, (S, 512))
        topk = topk_uniform(rng, T, S, k, cols, P0)
        ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.0625)
        out, lse = R.pertoken(dev_bf16(q), dev_bf16(kv), dev_i32(topk), P0, 0.0625)
        check_attention(out, lse, ref_out, ref_lse, f"d512 per-token S={S} cols={cols}")


@pytest.mark.parametrize("H", [16, 128])
def test_latent512_score_jump(R, H):
    """The exact fallbacks at 512 dims: one late key per affected token scores far above the
    rest (as in test_large_score_jump_and_negative_scale)."""
    rng = np.random.default_rng(45 + H)
    T, S, P0 = 24, 200, 176
    q = normal_bf16(rng, (T, H, 512))
    kv = normal_bf16(rng, (S, 512))
    topk = topk_uniform(rng, T, S, 120, 128, P0)
    for t in range(0, T, 3):
        r = t
        kv[r] = np.where(q[t, 0] & 0x8000, 0xC000, 0x4000).astype(np.uint16)
        topk[t][topk[t] == r] = -1
        topk[t, 120] = r
    for scale in (0.0625, -0.0625):
        ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale)
        qd, kvd, tkd = dev_bf16(q), dev_bf16(kv), dev_i32(topk)
        out, lse = R.pertoken(qd, kvd, tkd, P0, scale)
        check_attention(out, lse, ref_out, ref_lse, f"d512 H={H} per-token score jump, scale {scale}")
        out, lse, _ = R.grouped(qd, kvd, tkd, P0, scale)
        check_attention(out, lse, ref_out, ref_lse, f"d512 H={H} grouped score jump, scale {scale}")


# ---------------------------------------------------------------------------
# masked dense MHA
# ---------------------------------------------------------------------------

MHA_CASES = [
    # (label, seed, T, S, H, k, cols, P0, mode, dn, dr)
    ("causal_ragged", 20, 150, 150, 2, 40, 45, 0, "locality", 256, 0),
    ("chunked_ctx", 21, 100, 230, 3, 64, 70, 130, "uniform", 256, 0),
    ("all_selected", 22, 70, 70, 1, 70, 80, 0, "uniform", 256, 0),
    # K = k_nope (192) || k_pe (64, shared by the heads)
    ("rope_causal_ragged", 24, 150, 150, 2, 40, 45, 0, "locality", 192, 64),
    ("rope_chunked_ctx", 25, 100, 230, 3, 64, 70, 130, "uniform", 192, 64),
    ("rope_all_selected", 26, 300, 300, 2, 300, 300, 0, "uniform", 192, 64),
    # (128, 64, 128): K = k_nope (128) || k_pe (64), v 128
    ("dsv_causal_ragged", 27, 150, 150, 3, 40, 45, 0, "locality", 128, 64),
    ("dsv_chunked_ctx", 28, 100, 230, 2, 64, 70, 130, "uniform", 128, 64),
    ("dsv_all_selected", 29, 280, 280, 1, 280, 290, 0, "uniform", 128, 64),
]


def mha_dv(dn):
    return 128 if dn == 128 else 256


@pytest.mark.parametrize("case", MHA_CASES, ids=[c[0] for c in MHA_CASES])
def test_masked_mha_parity(R, case):
    label, seed, T, S, H, k, cols, P0, mode, dn, dr = case
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (T, H, dn + dr))
    kn = normal_bf16(rng, (S, H, dn))
    kp = normal_bf16(rng, (S, dr)) if dr else None
    v = normal_bf16(rng, (S, H, mha_dv(dn)))
    topk = (topk_uniform(rng, T, S, k, cols, P0) if mode == "uniform"
            else topk_locality(rng, T, S, k, cols, 8, P0))
    topk = shuffle_rows(topk, seed)
    scale = 1.0 / 16.0
    out, lse, ws = R.masked_mha(dev_bf16(q), dev_bf16(kn), None if kp is None else dev_bf16(kp),
                                dev_bf16(v), dev_i32(topk), P0, scale)
    ref_out, ref_lse = oracle.masked_mha(q, kn, kp, v, topk, S, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, label)
    # the workspace holds exactly the bit-packed selection
    words = (S + 31) // 32
    bits = np.zeros((T, words), np.uint32)
    for t in range(T):
        for x in oracle.selected_positions(topk[t], S, P0 + t):
            bits[t, x // 32] |= np.uint32(1) << np.uint32(x % 32)
    np.testing.assert_array_equal(ws.cpu().numpy().view(np.uint32), bits)


DENSE_CASES = [
    # (label, seed, T, S, H, P0, dn, dr)
    ("causal_two_tiles", 30, 300, 300, 2, 0, 256, 0),
    ("chunked_ctx", 31, 100, 230, 3, 130, 256, 0),
    ("positions_past_S", 32, 70, 90, 1, 60, 256, 0),
    ("rope_causal", 33, 280, 280, 2, 0, 192, 64),
    ("rope_chunked_ctx", 34, 90, 300, 2, 210, 192, 64),
    ("dsv_causal", 36, 270, 270, 2, 0, 128, 64),
    ("dsv_chunked_ctx", 37, 80, 300, 3, 220, 128, 64),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_mha_parity(R, case):
    label, seed, T, S, H, P0, dn, dr = case
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (T, H, dn + dr))
    kn = normal_bf16(rng, (S, H, dn))
    kp = normal_bf16(rng, (S, dr)) if dr else None
    v = normal_bf16(rng, (S, H, mha_dv(dn)))
    scale = 1.0 / 16.0
    out, lse = R.dense_mha(dev_bf16(q), dev_bf16(kn), None if kp is None else dev_bf16(kp), dev_bf16(v),
                           P0, scale)
    ref_out, ref_lse = oracle.dense_causal_mha(q, kn, kp, v, S, P0, scale)
    check_attention(out, lse, ref_out, ref_lse, label)


@pytest.mark.parametrize("dn,dr", [(256, 0), (192, 64), (128, 64)])
def test_dense_mha_equals_masked_when_topk_covers_the_chunk(R, dn, dr):
    """q_pos_offset + T <= k: both kernels do the same arithmetic on the same keys, so the
    outputs agree bit for bit."""
    rng = np.random.default_rng(35 + dr + dn)
    T, P0, H = 520, 40, 2
    S = P0 + T
    q = dev_bf16(normal_bf16(rng, (T, H, dn + dr)))
    kn = dev_bf16(normal_bf16(rng, (S, H, dn)))
    kp = dev_bf16(normal_bf16(rng, (S, dr))) if dr else None
    v = dev_bf16(normal_bf16(rng, (S, H, mha_dv(dn))))
    topk = shuffle_rows(topk_uniform(rng, T, S, S, S, P0), 35)
    om, lm, _ = R.masked_mha(q, kn, kp, v, dev_i32(topk), P0, 0.0625)
    od, ld = R.dense_mha(q, kn, kp, v, P0, 0.0625)
    torch.cuda.synchronize()
    assert torch.equal(od, om)
    assert torch.equal(ld, lm)


@pytest.mark.parametrize("dn,dr", [(256, 0), (192, 64), (128, 64)])
def test_masked_and_dense_mha_score_jump(R, dn, dr):
    """A few keys score far above everything earlier in their token's row (key rows set to
    +-8 along the token's query on head 0: ~140 units of the base-2 exponent above the
    first tile's maximum, beyond the fast kernel's 2^64 reference range), so those rows go
    through the exact path; the other rows and head 1 stay on the fast path."""
    rng = np.random.default_rng(41 + dn)
    T, S, H, P0 = 300, 300, 2, 0
    q = normal_bf16(rng, (T, H, dn + dr))
    kn = normal_bf16(rng, (S, H, dn))
    kp = normal_bf16(rng, (S, dr)) if dr else None
    v = normal_bf16(rng, (S, H, mha_dv(dn)))
    topk = topk_uniform(rng, T, S, 64, 70, P0)
    for t, x in ((250, 200), (263, 131), (299, 298), (40, 33)):
        kn[x, 0] = np.where(q[t, 0, :dn] & 0x8000, 0xC100, 0x4100).astype(np.uint16)  # bf16 -8 / +8
        topk[t][topk[t] == x] = -1
        topk[t, 3] = x
    topk = shuffle_rows(topk, 41)
    qd, knd, vd = dev_bf16(q), dev_bf16(kn), dev_bf16(v)
    kpd = None if kp is None else dev_bf16(kp)
    out, lse, _ = R.masked_mha(qd, knd, kpd, vd, dev_i32(topk), P0, 0.0625)
    ref_out, ref_lse = oracle.masked_mha(q, kn, kp, v, topk, S, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, f"masked score jump ({dn}, {dr})")
    out, lse = R.dense_mha(qd, knd, kpd, vd, P0, 0.0625)
    ref_out, ref_lse = oracle.dense_causal_mha(q, kn, kp, v, S, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, f"dense score jump ({dn}, {dr})")


def test_masked_and_dense_mha_long_context(R):
    """Keys past position 65535 (a 70000-key context, 20 query tokens at its end)."""
    rng = np.random.default_rng(38)
    T, S, H = 20, 70000, 2
    P0 = S - T
    q = normal_bf16(rng, (T, H, 256))
    kn = normal_bf16(rng, (S, H, 256))
    v = normal_bf16(rng, (S, H, 256))
    topk = topk_uniform(rng, T, S, 2048, 2100, P0)
    out, lse, _ = R.masked_mha(dev_bf16(q), dev_bf16(kn), None, dev_bf16(v), dev_i32(topk), P0, 0.0625)
    ref_out, ref_lse = oracle.masked_mha(q, kn, None, v, topk, S, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "masked S=70000")
    out, lse = R.dense_mha(dev_bf16(q), dev_bf16(kn), None, dev_bf16(v), P0, 0.0625)
    ref_out, ref_lse = oracle.dense_causal_mha(q, kn, None, v, S, P0, 0.0625)
    check_attention(out, lse, ref_out, ref_lse, "dense S=70000")


def test_masked_mha_equals_pertoken_with_shared_heads(R):
    """Heads sharing K = V = X: masked MHA must equal per-token sparse attention over X."""
    rng = np.random.default_rng(23)
    T, S, H = 90, 130, 2
    X = normal_bf16(rng, (S, 256))
    shared = np.ascontiguousarray(np.repeat(X[:, None, :], H, axis=1))
    q = normal_bf16(rng, (T, H, 256))
    topk = topk_locality(rng, T, S, 50, 55, 8, S - T)
    out, lse, _ = R.masked_mha(dev_bf16(q), dev_bf16(shared), None, dev_bf16(shared), dev_i32(topk),
                               S - T, 0.0625)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(q, X, topk, S, S - T, 0.0625, d_v=256)
    check_attention(out, lse, ref_out, ref_lse, "masked == per-token")
