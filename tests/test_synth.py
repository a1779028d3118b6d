"""The seeded input generators (CPU only)."""

import json
import os

import numpy as np

from synth import CONFIGS, make_case
from synth.gen import bf16_bits_from_f32, bf16_bits_to_f32, topk_locality, topk_uniform

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.5, 1.0 + 2.0**-9, 0.0], np.float32)
    b = bf16_bits_from_f32(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    np.testing.assert_array_equal(bf16_bits_to_f32(b), np.array(
        [1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0, 0.0], np.float32))


def test_tiny_config_is_deterministic():
    a, b = make_case(CONFIGS["c1_tiny"]), make_case(CONFIGS["c1_tiny"])
    for f in ("q", "kv", "topk"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.q.shape == (64, 16, 576) and a.kv.shape == (64, 576) and a.topk.shape == (64, 32)
    # uniform top-32 from positions <= t, -1 padded where t < 32
    assert int((a.topk >= 0).sum()) == sum(min(32, t + 1) for t in range(64))


def _check_rows(topk, S, k, P0):
    for t in range(topk.shape[0]):
        row = topk[t]
        valid = row[row >= 0]
        n = min(k, P0 + t + 1)
        assert valid.size == n
        assert np.all(row[n:] == -1)
        assert np.unique(valid).size == n
        assert valid.max() <= P0 + t and valid.max() < S


def test_generators_respect_causality_and_budget():
    rng = np.random.default_rng(0)
    _check_rows(topk_uniform(rng, 100, 140, 30, 36, 40), 140, 30, 40)
    _check_rows(topk_locality(rng, 100, 140, 30, 36, 8, 40), 140, 30, 40)
    _check_rows(topk_locality(rng, 60, 60, 50, 50, 1, 0), 60, 50, 0)


def test_locality_union_matches_pages_statistic():
    gold = json.load(open(os.path.join(GOLDEN, "union_size_8tok_top2048.json")))
    G, k = gold["G"], gold["k"]
    T = S = 4096
    topk = topk_locality(np.random.default_rng(123), T, S, k, k, G)
    sizes = [np.unique(topk[g:g + G][topk[g:g + G] >= 0]).size for g in range(k + 64, T, G)]
    lo, hi = gold["accepted_range"]
    assert lo <= float(np.mean(sizes)) <= hi


def test_config_table():
    c5 = CONFIGS["c5_long"]
    assert (c5.S, c5.T, c5.q_pos_offset, c5.cols, c5.k) == (32768, 21504, 11264, 2176, 2048)
    assert CONFIGS["c2_dsv32"].G == 1 and CONFIGS["c2_dsv32"].H == 128
    c4 = CONFIGS["c4_masked_nope"]
    assert (c4.dn, c4.dr, c4.dv, c4.scale) == (256, 0, 256, 1.0 / 16.0)
    # the K concat the NoPE layout skips is T * H * 256 * 2 bytes = 134 MB per 16k chunk
    assert c4.T * c4.H * c4.dn * 2 == 134217728
