"""Routing choice (host logic, CPU only): the rule's boundaries, and agreement with the
committed MI355X crossover measurements of every routing."""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pick():
    from mla_prefill_amd import _lib
    return _lib.dsa_select_routing


def test_dense_when_the_chunk_fits_in_the_top_k(pick):
    assert pick(1024, 1024, 0, 16, 2048, 256) == "dense"
    assert pick(2048, 2048, 0, 128, 2048, 256) == "dense"
    assert pick(1000, 2000, 1000, 16, 2048, 256) == "dense"      # q_pos_offset + T = k
    assert pick(1049, 2049, 1000, 16, 2048, 256) == "masked"     # one position more
    assert pick(1024, 1024, 0, 16, 2048, 0) == "grouped"      # no MHA inputs


def test_masked_threshold_against_grouped(pick):
    # H 16: c = 2.4, k = 2048 -> mean causal keys <= 4915.2; a chunk from 0 has mean (L + 1) / 2
    assert pick(9829, 9829, 0, 16, 2048, 256) == "masked"
    assert pick(9831, 9831, 0, 16, 2048, 256) == "grouped"
    # H 32: c = 1.95 -> mean <= 3993.6
    assert pick(7986, 7986, 0, 32, 2048, 256) == "masked"
    assert pick(7988, 7988, 0, 32, 2048, 256) == "grouped"
    assert pick(16384, 16384, 0, 64, 2048, 256) == "grouped"


def test_masked_threshold_against_pertoken(pick):
    # H 128: c = 1.4 -> mean causal keys <= 2867.2
    assert pick(5733, 5733, 0, 128, 2048, 256) == "masked"
    assert pick(5735, 5735, 0, 128, 2048, 256) == "per-token"
    assert pick(8192, 8192, 0, 128, 2048, 0) == "per-token"
    # H 48: no grouped form (128 % 48 != 0); c = 3.4
    assert pick(13000, 13000, 0, 48, 2048, 256) == "masked"
    assert pick(16384, 16384, 0, 48, 2048, 256) == "per-token"
    assert pick(16384, 16384, 0, 48, 2048, 0) == "per-token"


def test_thresholds_of_the_dsv32_geometry(pick):
    # (128, 64, 128): c = 3.6 / 3.05 / 2.75 against grouped, 2.4 at H 128
    assert pick(14744, 14744, 0, 16, 2048, 128) == "masked"
    assert pick(14746, 14746, 0, 16, 2048, 128) == "grouped"
    assert pick(9829, 9829, 0, 128, 2048, 128) == "masked"
    assert pick(9831, 9831, 0, 128, 2048, 128) == "per-token"
    assert pick(22000, 22000, 0, 48, 2048, 128) == "masked"
    from mla_prefill_amd import _lib
    assert _lib.lib.dsa_select_routing(8192, 8192, 0, 16, 2048, 192) == -3


def test_chunked_context_and_positions_past_S(pick):
    # a long prefix: mean causal keys ~ q_pos_offset + T / 2
    assert pick(512, 30512, 30000, 16, 2048, 256) == "grouped"
    assert pick(512, 4512, 4000, 16, 2048, 256) == "masked"
    assert pick(512, 5512, 5000, 16, 2048, 256) == "grouped"
    # positions past S - 1 see S keys
    assert pick(100, 3000, 5000, 16, 2048, 256) == "masked"
    assert pick(100, 9000, 9000, 16, 2048, 256) == "grouped"


def test_heads_only_the_mha_forms_take(pick):
    from mla_prefill_amd import _lib
    assert pick(8192, 8192, 0, 8, 2048, 256) == "masked"
    assert pick(1024, 1024, 0, 8, 2048, 256) == "dense"
    assert pick(8192, 8192, 0, 256, 2048, 256) == "masked"
    for H in (8, 24, 256):
        assert _lib.lib.dsa_select_routing(8192, 8192, 0, H, 2048, 0) == -3
    assert pick(8192, 8192, 0, 8, 2048, 128) == "masked"


def test_errors():
    from mla_prefill_amd import _lib
    f = _lib.lib.dsa_select_routing
    for args in ((-1, 10, 0, 16, 2048, 1), (10, 0, 0, 16, 2048, 1), (10, 10, -1, 16, 2048, 1),
                 (10, 10, 0, 0, 2048, 1), (10, 10, 0, 16, 0, 1)):
        assert f(*args) == -2
    assert f(0, 10, 0, 16, 2048, 0) == 3   # an empty chunk still names a routing (grouped)


def measured_rows():
    """(mha_dv, H, L, {routing: ms}) of every measured point; mha_dv from the section headers."""
    text = open(os.path.join(ROOT, "profiles", "crossover_mi355x.md")).read()
    rows = []
    mha_dv = None
    for line in text.splitlines():
        h = re.match(r"##.*\(mha_dv = (\d+)\)", line)
        if h:
            mha_dv = int(h.group(1))
        m = re.match(r"\|\s*(\d+)\s*\|\s*(\d+)\s*\|(.*)\|\s*([\w-]+)\s*\|$", line)
        if m:
            cells = [c.strip() for c in m.group(3).split("|")]
            ms = {name: float(c) for name, c in zip(("dense", "masked", "grouped", "per-token"), cells)
                  if c != "-"}
            rows.append((mha_dv, int(m.group(1)), int(m.group(2)), ms))
    return rows


def test_choice_is_near_the_fastest_measured_routing(pick):
    """At every measured point (both latent widths, both MHA value widths) the chosen routing is
    the fastest or within 10 % of it."""
    rows = measured_rows()
    assert len(rows) >= 110 and {r[0] for r in rows} == {256, 128}
    for mha_dv, H, L, ms in rows:
        choice = pick(L, L, 0, H, 2048, mha_dv)
        assert choice in ms, (mha_dv, H, L, choice)
        assert ms[choice] <= 1.10 * min(ms.values()), (mha_dv, H, L, choice, ms)
