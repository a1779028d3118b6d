"""Pins of the CPU oracle against things other than itself (CPU only).

* library routines: torch scaled_dot_product_attention / logsumexp in float64
  with a boolean mask built here from the selection rule with torch scatter;
* the textbook special case: all causal positions selected -> causal attention;
* closed forms: q = 0, a single selected row, n identical selected rows,
  empty selection;
* brute-force set arithmetic (pure Python) for the union list and mask;
* invariants: row permutation, -1 placement, wider buffers, non-causal and
  out-of-range entries, perturbing unselected rows, grouped == per-token,
  masked MHA == per-token MQA when all heads share K = V.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth.gen import normal_bf16, shuffle_rows, topk_locality, topk_uniform, widen


def to_t64(bits):
    """bf16 bits -> torch float64 through torch's own bfloat16 type."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def allowed_mask(topk, S, P0):
    """[T, S] bool: x appears in row t, 0 <= x < S, x <= P0 + t (built with torch scatter)."""
    tk = torch.from_numpy(topk.astype(np.int64))
    T = tk.shape[0]
    valid = (tk >= 0) & (tk < S)
    m = torch.zeros(T, S + 1, dtype=torch.bool)
    m.scatter_(1, torch.where(valid, tk, torch.full_like(tk, S)), True)
    m = m[:, :S]
    causal = torch.arange(S)[None, :] <= (P0 + torch.arange(T))[:, None]
    return m & causal


def sdpa_reference(q_bits, kv_bits, topk, S, P0, scale, d_v):
    q = to_t64(q_bits)                 # [T, H, d]
    kv = to_t64(kv_bits)[:S]           # [S, d]
    allow = allowed_mask(topk, S, P0)  # [T, S]
    T, H, _ = q.shape
    out = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), kv[None].expand(H, S, -1), kv[None, :, :d_v].expand(H, S, -1),
        attn_mask=allow[None], scale=scale).transpose(0, 1)
    logits = torch.einsum("thd,sd->ths", q, kv) * scale
    logits = logits.masked_fill(~allow[:, None, :], -math.inf)
    lse = torch.logsumexp(logits, dim=-1)
    return out.numpy(), lse.numpy(), allow.any(dim=1).numpy()


def rand_case(seed, T=40, S=48, H=4, d=24, cols=12, P0=None, extra_junk=True):
    rng = np.random.default_rng(seed)
    P0 = S - T if P0 is None else P0
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    topk = topk_uniform(rng, T, S, cols - 3 if extra_junk else cols, cols, P0)
    if extra_junk:
        # sprinkle entries the selection rule must ignore: -7, >= S, non-causal
        for t in range(T):
            row = topk[t]
            free = np.flatnonzero(row < 0)
            if free.size >= 3:
                p = P0 + t
                row[free[0]] = -7
                row[free[1]] = S + 3
                row[free[2]] = p + 1 if p + 1 < S else -1
    return q, kv, topk, P0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pertoken_matches_torch_sdpa(seed):
    S, T, d, dv = 48, 40, 24, 16
    q, kv, topk, P0 = rand_case(seed, T=T, S=S, d=d)
    scale = 0.37
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, scale, d_v=dv)
    ref_out, ref_lse, nonempty = sdpa_reference(q, kv, topk, S, P0, float(np.float32(scale)), dv)
    assert nonempty.all()
    np.testing.assert_allclose(out, ref_out, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_pertoken_without_rope_part_matches_torch_sdpa():
    # the 512-wide latent: scores and values over the same whole row (d_qk = d_v)
    S, T, d = 40, 33, 16
    q, kv, topk, P0 = rand_case(3, T=T, S=S, d=d)
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.29, d_v=d)
    ref_out, ref_lse, nonempty = sdpa_reference(q, kv, topk, S, P0, float(np.float32(0.29)), d)
    assert nonempty.all()
    np.testing.assert_allclose(out, ref_out, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_all_causal_selected_is_causal_attention():
    rng = np.random.default_rng(5)
    T = S = 33
    H, d, dv = 3, 20, 12
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    topk = widen(topk_uniform(rng, T, S, S, S), S + 5)   # k >= S: every causal position
    out, _ = oracle.pertoken_sparse_mqa(q, kv, topk, S, 0, 0.25, d_v=dv)
    qt, kt = to_t64(q).transpose(0, 1), to_t64(kv)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt[None].expand(H, S, d), kt[None, :, :dv].expand(H, S, dv),
        is_causal=True, scale=0.25).transpose(0, 1).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_closed_form_zero_query_is_mean_of_selected_values():
    rng = np.random.default_rng(7)
    T, S, H, d, dv = 6, 30, 2, 16, 8
    q = np.zeros((T, H, d), np.uint16)        # +0.0 in bf16
    kv = normal_bf16(rng, (S, d))
    topk = topk_uniform(rng, T, S, 5, 9, q_pos_offset=S - T)
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, S - T, 0.5, d_v=dv)
    kvf = to_t64(kv).numpy()
    for t in range(T):
        sel = [x for x in topk[t] if x >= 0]
        np.testing.assert_allclose(out[t], np.tile(kvf[sel, :dv].mean(0), (H, 1)), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[t], math.log(len(sel)), rtol=0, atol=1e-13)


def test_closed_form_single_selected_row():
    rng = np.random.default_rng(8)
    T, S, H, d, dv = 5, 20, 3, 24, 16
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    topk = np.full((T, 4), -1, np.int32)
    picks = [0, 3, 17, 9, 19]
    topk[:, 2] = picks
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, S - T, 0.125, d_v=dv)
    qf, kvf = to_t64(q).numpy(), to_t64(kv).numpy()
    for t, x in enumerate(picks):
        np.testing.assert_array_equal(out[t], np.tile(kvf[x, :dv], (H, 1)))
        # the dot product runs over the whole row (all d dims, including the rope part)
        np.testing.assert_allclose(lse[t], 0.125 * (qf[t] @ kvf[x]), rtol=1e-13, atol=1e-13)


def test_closed_form_identical_rows():
    rng = np.random.default_rng(9)
    T, S, H, d, dv = 1, 16, 2, 8, 4
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    kv[[2, 5, 11, 12]] = kv[7]
    topk = np.array([[5, -1, 2, 12, 7, 11]], np.int32)
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, S - 1, 0.3, d_v=dv)
    qf, kvf = to_t64(q).numpy(), to_t64(kv).numpy()
    s = float(np.float32(0.3)) * (qf[0] @ kvf[7])
    np.testing.assert_allclose(lse[0], s + math.log(5), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out[0], np.tile(kvf[7, :dv], (H, 1)), rtol=1e-13)


def test_empty_selection():
    rng = np.random.default_rng(10)
    T, S, H, d = 4, 8, 2, 8
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    topk = np.array([[-1, -1], [9, -3], [3, -1], [2, 5]], np.int32)  # rows 0-2 select nothing valid
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, 0, 1.0, d_v=4)
    for t in range(3):
        assert np.all(out[t] == 0) and np.all(np.isneginf(lse[t]))
    assert np.all(np.isfinite(lse[3]))


def test_duplicates_are_rejected():
    with pytest.raises(ValueError):
        oracle.selected_positions(np.array([3, 1, 3, -1]), 10, 9)


def test_invariances():
    S, T = 48, 40
    q, kv, topk, P0 = rand_case(11, T=T, S=S)
    base_out, base_lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.3, d_v=16)
    for variant in (shuffle_rows(topk, 1), widen(topk, 20), shuffle_rows(widen(topk, 17), 2)):
        o, l = oracle.pertoken_sparse_mqa(q, kv, variant, S, P0, 0.3, d_v=16)
        np.testing.assert_allclose(o, base_out, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l, base_lse, rtol=1e-13, atol=1e-13)
    # perturbing rows outside sel(t) leaves token t unchanged
    t = 17
    sel = set(oracle.selected_positions(topk[t], S, P0 + t).tolist())
    kv2 = kv.copy()
    for x in range(S):
        if x not in sel:
            kv2[x] = kv2[x] ^ np.uint16(0x1234)
    o, l = oracle.pertoken_sparse_mqa(q, kv2, topk, S, P0, 0.3, d_v=16, tokens=[t])
    np.testing.assert_array_equal(o[0], base_out[t])
    np.testing.assert_array_equal(l[0], base_lse[t])


# ---------------------------------------------------------------------------
# union list + mask: brute force with Python sets and invariants
# ---------------------------------------------------------------------------

def brute_union(topk, S, P0, G):
    T, cols = topk.shape
    pad = ((G * cols + 63) // 64) * 64
    NG = (T + G - 1) // G
    ui = [[-1] * pad for _ in range(NG)]
    ul = [0] * NG
    mk = [[0] * pad for _ in range(NG)]
    for g in range(NG):
        sets = []
        for t in range(g * G, min(T, g * G + G)):
            sets.append({int(x) for x in topk[t] if 0 <= x < S and x <= P0 + t})
        U = sorted(set().union(*sets))
        ul[g] = len(U)
        for j, x in enumerate(U):
            ui[g][j] = x
            mk[g][j] = sum(1 << i for i, s in enumerate(sets) if x in s)
    return np.array(ui, np.int32), np.array(ul, np.int32), np.array(mk, np.uint8)


@pytest.mark.parametrize("G,T,S,cols,P0,seed", [
    (8, 37, 45, 9, 8, 0), (4, 21, 21, 7, 0, 1), (2, 9, 30, 12, 21, 2), (1, 13, 13, 5, 0, 3),
    (8, 8, 64, 16, 56, 4), (3, 10, 10, 4, 0, 5),
])
def test_union_matches_brute_force(G, T, S, cols, P0, seed):
    rng = np.random.default_rng(seed)
    topk = topk_uniform(rng, T, S, max(1, cols - 2), cols, P0)
    topk[0, -1] = S + 1     # ignored: out of range
    topk[-1, -1] = -5       # ignored: negative
    ui, ul, mk = oracle.group_union_mask(topk, S, P0, G)
    bi, bl, bm = brute_union(topk, S, P0, G)
    np.testing.assert_array_equal(ui, bi)
    np.testing.assert_array_equal(ul, bl)
    np.testing.assert_array_equal(mk, bm)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_union_invariants(G):
    rng = np.random.default_rng(20 + G)
    T, S, k, cols, P0 = 203, 300, 64, 70, 97
    topk = shuffle_rows(topk_locality(rng, T, S, k, cols, G, P0), 3)
    ui, ul, mk = oracle.group_union_mask(topk, S, P0, G)
    pad = oracle.union_pad(G, cols)
    assert ui.shape == (-(-T // G), pad)
    for g in range(ui.shape[0]):
        n = int(ul[g])
        U = ui[g, :n]
        assert np.all(np.diff(U) > 0)                      # strictly ascending
        assert np.all(ui[g, n:] == -1) and np.all(mk[g, n:] == 0)
        assert n <= min(G * cols, P0 + g * G + G)
        for i, t in enumerate(range(g * G, min(T, g * G + G))):
            sel = oracle.selected_positions(topk[t], S, P0 + t)
            assert set(sel.tolist()) <= set(U.tolist())      # union covers every member
            assert int(((mk[g, :n] >> i) & 1).sum()) == sel.size
        last = min(T, g * G + G) - g * G
        assert np.all(mk[g, :n] >> last == 0)                # absent tokens have no bits
        if G == 1:
            sel = oracle.selected_positions(topk[g], S, P0 + g)
            np.testing.assert_array_equal(U, np.sort(sel))
            assert np.all(mk[g, :n] == 1)


def test_union_pad_formula():
    assert oracle.union_pad(8, 2048) == 16384
    assert oracle.union_pad(8, 2176) == 17408
    assert oracle.union_pad(1, 2048) == 2048
    assert oracle.union_pad(8, 32) == 256
    assert oracle.union_pad(3, 7) == 64


# ---------------------------------------------------------------------------
# grouped == per-token
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,T", [(16, 29), (32, 13), (64, 7), (128, 5)])
def test_grouped_equals_pertoken(H, T):
    rng = np.random.default_rng(H + T)
    G = 128 // H
    S, d, dv, cols = 40, 20, 12, 10
    P0 = S - T
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    topk = shuffle_rows(topk_locality(rng, T, S, 8, cols, G, P0), 4)
    ui, ul, mk = oracle.group_union_mask(topk, S, P0, G)
    og, lg = oracle.grouped_sparse_mqa(q, kv, ui, ul, mk, 0.2, d_v=dv)
    op, lp = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.2, d_v=dv)
    np.testing.assert_allclose(og, op, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lg, lp, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# masked dense MHA
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dr", [0, 6])
def test_masked_mha_matches_torch_sdpa(dr):
    rng = np.random.default_rng(30 + dr)
    T, S, H, dn, dv, cols = 22, 30, 3, 10, 7, 9
    P0 = S - T
    q = normal_bf16(rng, (T, H, dn + dr))
    kn = normal_bf16(rng, (S, H, dn))
    kp = normal_bf16(rng, (S, dr)) if dr else None
    v = normal_bf16(rng, (S, H, dv))
    topk = topk_uniform(rng, T, S, 6, cols, P0)
    out, lse = oracle.masked_mha(q, kn, kp, v, topk, S, P0, 0.4, )
    qt = to_t64(q).transpose(0, 1)                                  # [H, T, d]
    K = to_t64(kn).transpose(0, 1)                                  # [H, S, dn]
    if dr:
        K = torch.cat([K, to_t64(kp)[None].expand(H, S, dr)], dim=-1)
    V = to_t64(v).transpose(0, 1)
    allow = allowed_mask(topk, S, P0)
    sc = float(np.float32(0.4))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, K, V, attn_mask=allow[None], scale=sc)
    logits = (qt @ K.transpose(1, 2) * sc).masked_fill(~allow[None], -math.inf)
    np.testing.assert_allclose(out, ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).transpose(0, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_masked_mha_all_selected_is_causal():
    rng = np.random.default_rng(41)
    T = S = 25
    H, dn, dv = 2, 8, 8
    q = normal_bf16(rng, (T, H, dn))
    kn = normal_bf16(rng, (S, H, dn))
    v = normal_bf16(rng, (S, H, dv))
    topk = topk_uniform(rng, T, S, S, S)
    out, _ = oracle.masked_mha(q, kn, None, v, topk, S, 0, 0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        to_t64(q).transpose(0, 1), to_t64(kn).transpose(0, 1), to_t64(v).transpose(0, 1),
        is_causal=True, scale=0.5).transpose(0, 1).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_masked_mha_equals_pertoken_when_heads_share_kv():
    rng = np.random.default_rng(42)
    T, S, H, d, cols = 19, 26, 4, 12, 8
    P0 = S - T
    q = normal_bf16(rng, (T, H, d))
    X = normal_bf16(rng, (S, d))
    shared = np.repeat(X[:, None, :], H, axis=1)
    topk = topk_locality(rng, T, S, 6, cols, 8, P0)
    om, lm = oracle.masked_mha(q, shared, None, shared, topk, S, P0, 0.3)
    op, lp = oracle.pertoken_sparse_mqa(q, X, topk, S, P0, 0.3, d_v=d)
    np.testing.assert_allclose(om, op, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lm, lp, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# dense causal MHA (the shortcut for chunks no longer than the top-k)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dr,P0", [(0, 0), (5, 7), (5, 40)])
def test_dense_mha_matches_torch_sdpa(dr, P0):
    # causal mask with the chunk offset built from torch.tril; P0 = 40 puts the
    # last positions past S - 1 (they see every key)
    rng = np.random.default_rng(50 + dr + P0)
    T, S, H, dn, dv = 21, 33, 3, 9, 6
    q = normal_bf16(rng, (T, H, dn + dr))
    kn = normal_bf16(rng, (S, H, dn))
    kp = normal_bf16(rng, (S, dr)) if dr else None
    v = normal_bf16(rng, (S, H, dv))
    out, lse = oracle.dense_causal_mha(q, kn, kp, v, S, P0, 0.35)
    qt = to_t64(q).transpose(0, 1)
    K = to_t64(kn).transpose(0, 1)
    if dr:
        K = torch.cat([K, to_t64(kp)[None].expand(H, S, dr)], dim=-1)
    V = to_t64(v).transpose(0, 1)
    allow = torch.ones(T, S, dtype=torch.bool).tril(P0)
    sc = float(np.float32(0.35))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, K, V, attn_mask=allow[None], scale=sc)
    logits = (qt @ K.transpose(1, 2) * sc).masked_fill(~allow[None], -math.inf)
    np.testing.assert_allclose(out, ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).transpose(0, 1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P0", [0, 6])
def test_dense_mha_equals_masked_when_topk_covers_the_chunk(P0):
    # the shortcut's premise: with q_pos_offset + T <= k every causal key is in the top-k
    rng = np.random.default_rng(60 + P0)
    T, H, d = 18, 2, 8
    S = P0 + T
    q = normal_bf16(rng, (T, H, d))
    kn = normal_bf16(rng, (S, H, d))
    v = normal_bf16(rng, (S, H, d))
    topk = topk_uniform(rng, T, S, S, S + 3, P0)   # every causal position, shuffled, -1 padded
    om, lm = oracle.masked_mha(q, kn, None, v, topk, S, P0, 0.5)
    od, ld = oracle.dense_causal_mha(q, kn, None, v, S, P0, 0.5)
    np.testing.assert_allclose(od, om, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ld, lm, rtol=1e-12, atol=1e-13)


def test_dense_mha_first_position_sees_one_key():
    rng = np.random.default_rng(63)
    T = S = 5
    H, d = 2, 4
    q = normal_bf16(rng, (T, H, d))
    kn = normal_bf16(rng, (S, H, d))
    v = normal_bf16(rng, (S, H, d))
    out, lse = oracle.dense_causal_mha(q, kn, None, v, S, 0, 0.25, tokens=[0])
    qq, kk, vv = (oracle.bf16_to_f64(a) for a in (q, kn, v))
    np.testing.assert_array_equal(out[0], vv[0])
    sc = float(np.float32(0.25))
    np.testing.assert_allclose(lse[0], sc * np.einsum("hd,hd->h", qq[0], kk[0]), rtol=1e-14)


# ---------------------------------------------------------------------------
# FP8 KV latent
# ---------------------------------------------------------------------------

def test_fp8_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.fp8_e4m3_to_f64(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_fp8_decode_closed_forms():
    v = oracle.fp8_e4m3_to_f64(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0xB8, 0x7F, 0xFF],
                                        np.uint8))
    assert v[0] == 0 and v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 1.0 and v[5] == 1.5 and v[6] == 448.0 and v[7] == -1.0
    assert np.isnan(v[8]) and np.isnan(v[9])


@pytest.mark.parametrize("per_row", [False, True])
def test_fp8_dequant_is_the_exact_product(per_row):
    """e4m3 * scale in float64 is exact (4 significant bits times 24): it equals torch's
    float8_e4m3fn decode times the float32 scale computed in float64, bit for bit."""
    rng = np.random.default_rng(71 + per_row)
    S, d = 37, 40
    kv8 = rng.integers(0, 256, (S, d)).astype(np.uint8)
    kv8[(kv8 & 0x7F) == 0x7F] = 0x3A   # no NaN codes in a cache
    scale = (rng.uniform(0.01, 3.0, S) if per_row else np.float32(0.0371)).astype(np.float32)
    f = torch.from_numpy(kv8).view(torch.float8_e4m3fn).double()
    sc = torch.from_numpy(np.atleast_1d(scale)).double()
    prod = f * (sc[:, None] if per_row else sc[0])
    np.testing.assert_array_equal(oracle.dequant_latent_fp8(kv8, scale), prod.numpy())


def test_fp8_attention_matches_torch_sdpa_on_scaled_rows():
    """Per-row scales that are not powers of two (the scaled elements are not bf16 numbers):
    the oracle equals torch SDPA / logsumexp in float64 over torch's own decode of the codes
    times the scales, under the selection mask built with torch scatter."""
    rng = np.random.default_rng(75)
    T, S, H, d, dv = 30, 41, 3, 24, 16
    kv8 = rng.integers(0, 256, (S, d)).astype(np.uint8)
    kv8[(kv8 & 0x7F) == 0x7F] = 0x33
    scale_kv = rng.uniform(0.003, 0.9, S).astype(np.float32)
    q = normal_bf16(rng, (T, H, d))
    topk = topk_uniform(rng, T, S, 9, 11, S - T)
    topk[3, -1] = S + 4          # out of range: ignored
    sc = float(np.float32(0.31))
    out, lse = oracle.pertoken_sparse_mqa_fp8(q, kv8, scale_kv, topk, S, S - T, 0.31, d_v=dv)
    kv = torch.from_numpy(kv8).view(torch.float8_e4m3fn).double() * torch.from_numpy(scale_kv).double()[:, None]
    qt = to_t64(q)
    allow = allowed_mask(topk, S, S - T)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt.transpose(0, 1), kv[None].expand(H, S, -1), kv[None, :, :dv].expand(H, S, -1),
        attn_mask=allow[None], scale=sc).transpose(0, 1)
    logits = torch.einsum("thd,sd->ths", qt, kv) * sc
    ref_lse = torch.logsumexp(logits.masked_fill(~allow[:, None, :], -math.inf), dim=-1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_fp8_attention_equals_bf16_attention_on_exact_values():
    """A power-of-two scale keeps every scaled element a bf16 number, so the FP8 definition
    must equal the (pinned) bf16 one on those bits; per-row scales all equal to it as well."""
    from synth.gen import bf16_bits_from_f32
    rng = np.random.default_rng(73)
    T, S, H, d, dv = 20, 30, 2, 24, 16
    kv8 = rng.integers(0, 256, (S, d)).astype(np.uint8)
    kv8[(kv8 & 0x7F) == 0x7F] = 0x41
    q = normal_bf16(rng, (T, H, d))
    topk = topk_uniform(rng, T, S, 8, 10, S - T)
    sc = np.float32(0.125)
    vals = torch.from_numpy(kv8).view(torch.float8_e4m3fn).float().numpy() * sc
    kv_bits = bf16_bits_from_f32(vals)
    np.testing.assert_array_equal(oracle.bf16_to_f64(kv_bits), vals.astype(np.float64))   # exact in bf16
    ref = oracle.pertoken_sparse_mqa(q, kv_bits, topk, S, S - T, 0.3, d_v=dv)
    for scale_kv in (sc, np.full(S, sc, np.float32)):
        got = oracle.pertoken_sparse_mqa_fp8(q, kv8, scale_kv, topk, S, S - T, 0.3, d_v=dv)
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])


def test_fp8_paged_equals_single_sequence_on_gathered_rows():
    """A paged FP8 batch of one request equals the single-sequence FP8 definition over the
    request's rows gathered in position order (codes and scales moved together)."""
    rng = np.random.default_rng(76)
    T, P0, H, d, page = 9, 14, 2, 24, 4
    L = P0 + T
    pages = -(-L // page)
    perm = rng.permutation(pages + 2).astype(np.int32)
    bt = perm[:pages][None]
    ns = (pages + 2) * page
    cache8 = rng.integers(0, 0x7E, (ns, d)).astype(np.uint8)
    sck = rng.uniform(0.01, 2.0, ns).astype(np.float32)
    q = normal_bf16(rng, (T, H, d))
    topk = topk_uniform(rng, T, L, 6, 7, P0)
    got = oracle.pertoken_sparse_mqa_varlen_fp8(q, cache8, sck, topk, np.array([0, T]), np.array([L]),
                                                np.array([P0]), bt, page, 0.2, d_v=16)
    rows = np.array([oracle.physical_row(bt, 0, x, page) for x in range(L)])
    ref = oracle.pertoken_sparse_mqa_fp8(q, cache8[rows], sck[rows], topk, L, P0, 0.2, d_v=16)
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1], ref[1])


def test_fp8_per_row_scale_scales_values_only():
    """Doubling one row's scale doubles that row's value vector and its dot products: with the
    row as the only selection, out doubles and LSE moves by scale * q.k."""
    rng = np.random.default_rng(74)
    S, d = 6, 16
    kv8 = rng.integers(0, 0x70, (S, d)).astype(np.uint8)
    q = normal_bf16(rng, (1, 1, d))
    topk = np.array([[4, -1]], np.int32)
    s1 = np.full(S, 0.5, np.float32)
    s2 = s1.copy()
    s2[4] = 1.0
    o1, l1 = oracle.pertoken_sparse_mqa_fp8(q, kv8, s1, topk, S, S - 1, 0.2, d_v=8)
    o2, l2 = oracle.pertoken_sparse_mqa_fp8(q, kv8, s2, topk, S, S - 1, 0.2, d_v=8)
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-14)
    qk = oracle.bf16_to_f64(q[0, 0]) @ oracle.fp8_e4m3_to_f64(kv8[4])
    np.testing.assert_allclose(l1[0, 0], float(np.float32(0.2)) * 0.5 * qk, rtol=1e-12)
    np.testing.assert_allclose(l2[0, 0], float(np.float32(0.2)) * 1.0 * qk, rtol=1e-12)


# ---------------------------------------------------------------------------
# batches of requests over a paged KV cache
# ---------------------------------------------------------------------------

def _varlen_args(c):
    return (c.cu_seqlens, c.kv_lens, c.q_pos_start, c.block_table, c.page_size)


def test_varlen_single_request_identity_pages_reduces_to_plain():
    """One request whose page table is the identity: the paged functions equal the
    single-sequence ones exactly (same rows in the same order)."""
    rng = np.random.default_rng(40)
    T, S, P0, H, d, page, G = 21, 44, 23, 2, 24, 4, 8
    q = normal_bf16(rng, (T, H, d))
    kv = normal_bf16(rng, (S, d))
    topk = shuffle_rows(widen(topk_locality(rng, T, S, 9, 9, G, P0), 12), 40)
    cu, kvl, p0 = np.array([0, T]), np.array([S]), np.array([P0])
    bt = np.arange(S // page, dtype=np.int32)[None]
    out_v, lse_v = oracle.pertoken_sparse_mqa_varlen(q, kv, topk, cu, kvl, p0, bt, page, 0.3, d_v=16)
    out, lse = oracle.pertoken_sparse_mqa(q, kv, topk, S, P0, 0.3, d_v=16)
    np.testing.assert_array_equal(out_v, out)
    np.testing.assert_array_equal(lse_v, lse)
    ng = -(-T // G)
    info, ui, ul, mk = oracle.group_union_mask_varlen(topk, cu, kvl, p0, bt, page, S, G, ng + 2)
    ui0, ul0, mk0 = oracle.group_union_mask(topk, S, P0, G)
    np.testing.assert_array_equal(ui[:ng], ui0)
    np.testing.assert_array_equal(ul[:ng], ul0)
    np.testing.assert_array_equal(mk[:ng], mk0)
    assert (ul[ng:] == 0).all() and (ui[ng:] == -1).all() and (info[ng:] == 0).all()
    np.testing.assert_array_equal(info[:ng], [(g * G, min(G, T - g * G)) for g in range(ng)])


def _permute_pages(c, perm):
    """The same batch with physical page p moved to perm[p]."""
    ps = c.page_size
    cache = np.empty_like(c.kv_cache)
    for p in range(c.kv_cache.shape[0] // ps):
        cache[perm[p] * ps:(perm[p] + 1) * ps] = c.kv_cache[p * ps:(p + 1) * ps]
    bt = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    return cache, bt


def test_varlen_page_placement_does_not_matter():
    from synth import make_varlen_case
    c = make_varlen_case(41, [7, 19, 1, 12], [0, 30, 5, 17], H=2, k=10, cols=13, page_size=4,
                         d_qk=24)
    perm = np.random.default_rng(41).permutation(c.kv_cache.shape[0] // c.page_size)
    cache2, bt2 = _permute_pages(c, perm)
    a = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *_varlen_args(c), 0.25, d_v=16)
    b = oracle.pertoken_sparse_mqa_varlen(c.q, cache2, c.topk, c.cu_seqlens, c.kv_lens,
                                          c.q_pos_start, bt2, c.page_size, 0.25, d_v=16)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    mg = c.max_groups()
    u1 = oracle.group_union_mask_varlen(c.topk, *_varlen_args(c), c.num_slots, c.G, mg)
    u2 = oracle.group_union_mask_varlen(c.topk, c.cu_seqlens, c.kv_lens, c.q_pos_start, bt2,
                                        c.page_size, c.num_slots, c.G, mg)
    ps = c.page_size
    moved = np.where(u1[1] >= 0, perm[np.maximum(u1[1], 0) // ps] * ps + np.maximum(u1[1], 0) % ps, -1)
    np.testing.assert_array_equal(u2[1], moved)
    for i in (0, 2, 3):
        np.testing.assert_array_equal(u1[i], u2[i])


def test_varlen_batch_equals_each_request_alone():
    from synth import make_varlen_case
    c = make_varlen_case(42, [9, 3, 14], [11, 0, 6], H=2, k=8, cols=8, page_size=8, d_qk=24)
    out, lse = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *_varlen_args(c), 0.2, d_v=16)
    for r in range(c.cu_seqlens.size - 1):
        a, b = int(c.cu_seqlens[r]), int(c.cu_seqlens[r + 1])
        o1, l1 = oracle.pertoken_sparse_mqa_varlen(
            c.q[a:b], c.kv_cache, c.topk[a:b], np.array([0, b - a]), c.kv_lens[r:r + 1],
            c.q_pos_start[r:r + 1], c.block_table[r:r + 1], c.page_size, 0.2, d_v=16)
        np.testing.assert_array_equal(o1, out[a:b])
        np.testing.assert_array_equal(l1, lse[a:b])


@pytest.mark.parametrize("mode", ["locality", "uniform"])
def test_varlen_grouped_equals_pertoken(mode):
    from synth import make_varlen_case
    c = make_varlen_case(43, [13, 1, 8, 17], [20, 3, 0, 9], H=4, k=12, cols=15, page_size=4,
                         G=4, mode=mode, d_qk=24)
    mg = c.max_groups() + 3
    info, ui, ul, mk = oracle.group_union_mask_varlen(c.topk, *_varlen_args(c), c.num_slots, c.G, mg)
    og, lg = oracle.grouped_sparse_mqa_varlen(c.q, c.kv_cache, info, ui, ul, mk, 0.3, d_v=16)
    op, lp = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *_varlen_args(c), 0.3, d_v=16)
    np.testing.assert_allclose(og, op, rtol=0, atol=1e-12)
    fin = np.isfinite(lp)
    np.testing.assert_array_equal(np.isfinite(lg), fin)
    np.testing.assert_allclose(lg[fin], lp[fin], rtol=0, atol=1e-12)


def test_varlen_convert_then_single_sequence_equals_varlen():
    """Physical-row top-k (the index conversion) fed to the single-sequence per-token
    function over the whole cache, with causality already applied, equals the paged one."""
    from synth import make_varlen_case
    c = make_varlen_case(44, [6, 11, 4], [9, 0, 30], H=2, k=7, cols=9, page_size=4, d_qk=24)
    g = oracle.convert_req_index_to_global(c.topk, *_varlen_args(c), c.num_slots)
    n = c.num_slots
    a = oracle.pertoken_sparse_mqa(c.q, c.kv_cache, g, n, n - 1, 0.4, d_v=16)
    b = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *_varlen_args(c), 0.4, d_v=16)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # entries it drops: -1, beyond the request's KV, beyond the token's position
    owner = oracle.request_of_tokens(c.cu_seqlens)
    for t in range(g.shape[0]):
        r = owner[t]
        pos = c.q_pos_start[r] + t - c.cu_seqlens[r]
        for col in range(g.shape[1]):
            x = c.topk[t, col]
            assert (g[t, col] >= 0) == (0 <= x < c.kv_lens[r] and x <= pos)


def test_varlen_groups_stay_inside_requests():
    cu = np.array([0, 3, 3, 20, 21, 37])
    owner = oracle.request_of_tokens(cu)
    groups = oracle.varlen_groups(cu, 8)
    assert sum(n for _, n in groups) == 37
    assert len(groups) == sum(-(-int(n) // 8) for n in np.diff(cu))
    for t0, n in groups:
        assert 1 <= n <= 8 and owner[t0] == owner[t0 + n - 1]
        assert t0 == cu[owner[t0]] or (t0 - cu[owner[t0]]) % 8 == 0


def test_varlen_rows_outside_the_cache_are_ignored():
    from synth import make_varlen_case
    c = make_varlen_case(45, [10], [12], H=2, k=9, cols=9, page_size=4, d_qk=24, spare_pages=0)
    bt = c.block_table.copy()
    bt[0, 1] = c.num_slots // c.page_size + 5     # page 1 of the request points past the cache
    out, lse = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, c.cu_seqlens, c.kv_lens,
                                                 c.q_pos_start, bt, c.page_size, 0.5, d_v=16)
    topk2 = np.where((c.topk >= 4) & (c.topk < 8), -1, c.topk)  # the same positions dropped
    o2, l2 = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, topk2, *_varlen_args(c), 0.5, d_v=16)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)
