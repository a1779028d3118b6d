"""The C-ABI library: exports and host-side argument checks (CPU only).

Every call below is rejected on the host before any HIP call, so it runs
without a GPU.  No compute call is made here.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_prefill.h")
LIB = os.path.join(ROOT, "mla_prefill_amd", "libdsa_prefill.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdsa_prefill.so not built")

OK, NULL, SHAPE, UNSUP, ALIGN = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from mla_prefill_amd import _lib
    return _lib.lib


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("dsa_build_group_union", "dsa_sparse_prefill_grouped", "dsa_sparse_prefill_pertoken",
              "dsa_masked_mha_prefill"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dsa_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        getattr(lib, name)  # resolvable through the dynamic loader too


def test_binding_covers_every_declared_symbol():
    from mla_prefill_amd import _lib
    assert set(declared_functions()) == set(_lib.EXPORTED)


def test_helpers(lib):
    from mla_prefill_amd import _lib
    assert _lib.dsa_abi_version() == 2
    assert _lib.dsa_union_pad(8, 2048) == 16384
    assert _lib.dsa_union_pad(8, 2176) == 17408
    assert _lib.dsa_union_pad(1, 1) == 64
    assert lib.dsa_union_pad(0, 5) == SHAPE and lib.dsa_union_pad(9, 5) == SHAPE
    assert lib.dsa_union_pad(8, -1) == SHAPE and lib.dsa_union_pad(8, 2**30) == SHAPE
    assert _lib.dsa_masked_mha_workspace_bytes(16384, 16384) == 16384 * 512 * 4
    assert _lib.dsa_masked_mha_workspace_bytes(3, 33) == 3 * 2 * 4
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(_lib.dsa_status_string(s), str)


P = 0x10000  # a non-null, 16-byte aligned fake address: never dereferenced on these paths


def union_call(lib, topk=P, ld=32, T=64, cols=32, S=64, P0=0, G=8, pad=256, ui=P, ul=P, mk=P):
    return lib.dsa_build_group_union(topk, ld, T, cols, S, P0, G, pad, ui, ul, mk, None)


def test_union_validation(lib):
    assert union_call(lib, T=-1) == SHAPE
    assert union_call(lib, S=0) == SHAPE
    assert union_call(lib, ld=31) == SHAPE
    assert union_call(lib, P0=-1) == SHAPE
    assert union_call(lib, G=0) == SHAPE and union_call(lib, G=9) == SHAPE
    assert union_call(lib, pad=192) == SHAPE          # < G * cols
    assert union_call(lib, pad=257) == SHAPE          # not a multiple of 64
    assert union_call(lib, T=0) == OK                 # nothing to do, nothing enqueued
    assert union_call(lib, topk=None) == NULL
    assert union_call(lib, ui=None) == NULL
    assert union_call(lib, ul=None) == NULL
    assert union_call(lib, mk=None) == NULL
    assert union_call(lib, topk=P + 2) == ALIGN
    assert union_call(lib, ui=P + 1) == ALIGN


def grouped_call(lib, q=P, kv=P, ui=P, ul=P, mk=P, T=64, H=16, S=64, pad=256, dqk=576, dv=512,
                 out=P, lse=P, scale=0.1):
    return lib.dsa_sparse_prefill_grouped(q, kv, ui, ul, mk, T, H, S, pad, dqk, dv, scale, out, lse, None)


def test_grouped_validation(lib):
    for H in (8, 24, 48, 256):
        assert grouped_call(lib, H=H) == UNSUP
    assert grouped_call(lib, dqk=448) == UNSUP and grouped_call(lib, dv=256) == UNSUP
    assert grouped_call(lib, dqk=512, dv=576) == UNSUP
    assert grouped_call(lib, dqk=512, T=0) == OK       # the 512-wide latent (no rope part)
    assert grouped_call(lib, T=-3) == SHAPE and grouped_call(lib, S=0) == SHAPE
    assert grouped_call(lib, pad=48) == SHAPE          # union rows must hold whole 32-slot tiles
    assert grouped_call(lib, T=0) == OK
    for kw in ("q", "kv", "ui", "ul", "mk", "out", "lse"):
        assert grouped_call(lib, **{kw: None}) == NULL
    assert grouped_call(lib, q=P + 8) == ALIGN
    assert grouped_call(lib, kv=P + 2) == ALIGN
    assert grouped_call(lib, out=P + 4) == ALIGN
    assert grouped_call(lib, lse=P + 2) == ALIGN
    assert grouped_call(lib, mk=P + 2) == ALIGN        # membership bytes are read 4 at a time


def pertoken_call(lib, q=P, kv=P, tk=P, ld=32, T=64, H=16, S=64, cols=32, P0=0, dqk=576, dv=512,
                  out=P, lse=P, scale=0.1):
    return lib.dsa_sparse_prefill_pertoken(q, kv, tk, ld, T, H, S, cols, P0, dqk, dv, scale, out, lse, None)


def test_pertoken_validation(lib):
    for H in (8, 24, 136, 0):
        assert pertoken_call(lib, H=H) == UNSUP
    assert pertoken_call(lib, dqk=192) == UNSUP and pertoken_call(lib, dqk=512, dv=256) == UNSUP
    assert pertoken_call(lib, dqk=512, T=0) == OK
    assert pertoken_call(lib, ld=16) == SHAPE and pertoken_call(lib, cols=-1) == SHAPE
    assert pertoken_call(lib, P0=-5) == SHAPE
    assert pertoken_call(lib, T=0) == OK
    for kw in ("q", "kv", "tk", "out", "lse"):
        assert pertoken_call(lib, **{kw: None}) == NULL
    assert pertoken_call(lib, q=P + 2) == ALIGN and pertoken_call(lib, tk=P + 1) == ALIGN


def auto_call(lib, q=P, kv=P, tk=P, ld=32, T=64, H=16, S=64, cols=32, P0=0, dqk=576, dv=512, scale=0.0625,
              pad=256, ui=P, ul=P, mk=P, route=P, out=P, lse=P):
    return lib.dsa_sparse_prefill_auto(q, kv, tk, ld, T, H, S, cols, P0, dqk, dv, scale, pad, ui, ul, mk, route,
                                       out, lse, None)


def test_auto_validation(lib):
    for H in (128, 48, 8, 0):                       # only the head counts with a grouped form
        assert auto_call(lib, H=H) == UNSUP
    assert auto_call(lib, dqk=192) == UNSUP and auto_call(lib, scale=0.0) == UNSUP
    assert auto_call(lib, T=0) == OK
    assert auto_call(lib, ld=16) == SHAPE and auto_call(lib, P0=-1) == SHAPE
    assert auto_call(lib, pad=192) == SHAPE         # below G * cols = 256
    assert auto_call(lib, pad=288) == SHAPE         # not a multiple of 64
    for kw in ("q", "kv", "tk", "ui", "ul", "mk", "route", "out", "lse"):
        assert auto_call(lib, **{kw: None}) == NULL
    assert auto_call(lib, route=P + 2) == ALIGN and auto_call(lib, ul=P + 1) == ALIGN


def mha_call(lib, q=P, kn=P, kp=None, v=P, tk=P, ld=32, T=64, S=64, H=16, dn=256, dr=0, dv=256,
             cols=32, P0=0, ws=P, out=P, lse=P, scale=0.0625):
    return lib.dsa_masked_mha_prefill(q, kn, kp, v, tk, ld, T, S, H, dn, dr, dv, cols, P0, scale, ws,
                                      out, lse, None)


def test_masked_mha_validation(lib):
    # (192, 64, 256) needs k_pe; (256, 64, 256) and other head dims are not supported
    assert mha_call(lib, dn=192, dr=64) == NULL
    assert mha_call(lib, dn=192, dr=64, kp=P + 2) == ALIGN
    assert mha_call(lib, dn=192, dr=64, kp=P, T=0) == OK
    assert mha_call(lib, dn=256, dr=64) == UNSUP and mha_call(lib, dn=192, dr=64, dv=128) == UNSUP
    # (128, 64, 128): the DeepSeek-V3.2 geometry
    assert mha_call(lib, dn=128, dr=64, dv=128) == NULL
    assert mha_call(lib, dn=128, dr=64, dv=128, kp=P, T=0) == OK
    assert mha_call(lib, dn=128, dr=0, dv=128) == UNSUP and mha_call(lib, dn=128, dr=64, dv=256) == UNSUP
    assert mha_call(lib, dn=128) == UNSUP and mha_call(lib, dv=128) == UNSUP
    assert mha_call(lib, H=0) == SHAPE and mha_call(lib, ld=8) == SHAPE
    assert mha_call(lib, H=65537) == SHAPE and mha_call(lib, T=2**31 - 1, H=65536) == SHAPE
    assert mha_call(lib, T=0) == OK
    for kw in ("q", "kn", "v", "tk", "ws", "out", "lse"):
        assert mha_call(lib, **{kw: None}) == NULL
    assert mha_call(lib, kn=P + 2) == ALIGN and mha_call(lib, ws=P + 2) == ALIGN


def test_masked_mha_noalloc_validation(lib):
    """The no-allocation form: the same host checks without a workspace argument, and
    DSA_ERR_CAPACITY (checked before any HIP call) past the static scratch."""
    CAPACITY = -6
    def call(q=P, kn=P, kp=None, v=P, tk=P, ld=16, T=4, S=8, H=2, dn=256, dr=0, dv=256, cols=16, P0=0,
             scale=0.1, out=P, lse=P):
        return lib.dsa_masked_mha_prefill_noalloc(q, kn, kp, v, tk, ld, T, S, H, dn, dr, dv, cols, P0, scale,
                                                  out, lse, None)
    assert call(dn=192, dr=64) == NULL and call(dn=256, dr=64) == UNSUP and call(scale=0.0) == UNSUP
    assert call(H=0) == SHAPE and call(ld=8) == SHAPE and call(T=0) == OK
    for kw in ("q", "kn", "v", "tk", "out", "lse"):
        assert call(**{kw: None}) == NULL
    assert call(kn=P + 2) == ALIGN
    # 16384 x ceil(32800 / 32) words = 67 MB > 32 MiB; 16384 x 16384 fits exactly
    assert lib.dsa_masked_mha_workspace_bytes(16384, 16384) == 32 << 20
    assert call(T=16384, S=32800) == CAPACITY
    assert lib.dsa_status_string(CAPACITY).decode().startswith("the work needs more than")


def dense_call(lib, q=P, kn=P, kp=None, v=P, T=4, S=8, H=2, dn=256, dr=0, dv=256, p0=0, scale=0.1,
               out=P, lse=P):
    return lib.dsa_dense_mha_prefill(q, kn, kp, v, T, S, H, dn, dr, dv, p0, scale, out, lse, None)


def test_dense_mha_validation(lib):
    assert dense_call(lib, dn=192, dr=64) == NULL
    assert dense_call(lib, dn=192, dr=64, kp=P + 2) == ALIGN
    assert dense_call(lib, dn=192, dr=64, kp=P, T=0) == OK
    assert dense_call(lib, dn=256, dr=64) == UNSUP and dense_call(lib, dv=128) == UNSUP
    assert dense_call(lib, H=0) == SHAPE and dense_call(lib, S=0) == SHAPE and dense_call(lib, p0=-1) == SHAPE
    assert dense_call(lib, H=65537) == SHAPE and dense_call(lib, T=2**31 - 1, H=65536) == SHAPE
    assert dense_call(lib, T=0) == OK
    for kw in ("q", "kn", "v", "out", "lse"):
        assert dense_call(lib, **{kw: None}) == NULL
    assert dense_call(lib, q=P + 2) == ALIGN and dense_call(lib, lse=P + 2) == ALIGN
    for bad in (0.0, float("nan")):
        assert dense_call(lib, scale=bad) == UNSUP


def test_scale_must_be_finite_and_nonzero(lib):
    for bad in (0.0, -0.0, float("inf"), float("-inf"), float("nan")):
        assert grouped_call(lib, scale=bad) == UNSUP
        assert pertoken_call(lib, scale=bad) == UNSUP
        assert mha_call(lib, scale=bad) == UNSUP
    for good in (1e-30, -0.1, 3.0e30):
        assert grouped_call(lib, scale=good, T=0) == OK
        assert pertoken_call(lib, scale=good, T=0) == OK
        assert mha_call(lib, scale=good, T=0) == OK


def test_library_links_only_hip_runtime():
    out = subprocess.run(["ldd", LIB], capture_output=True, text=True).stdout
    assert "libamdhip64" in out
    assert "torch" not in out and "python" not in out


def test_varlen_validation(lib):
    assert lib.dsa_varlen_group_bound(37, 5, 8) == 10 and lib.dsa_varlen_group_bound(3, 5, 8) == 3
    assert lib.dsa_varlen_group_bound(0, 1, 8) == 0
    for args in ((-1, 1, 8), (5, 0, 8), (5, 1, 0), (5, 1, 9)):
        assert lib.dsa_varlen_group_bound(*args) == SHAPE
    def conv(tk=P, ld=16, T=8, cols=16, R_=2, cu=P, kl=P, qs=P, bt=P, bt_ld=4, ps=64, ns=256, out=P):
        return lib.dsa_convert_req_index_to_global(tk, ld, T, cols, R_, cu, kl, qs, bt, bt_ld, ps, ns, out, None)
    assert conv(R_=0) == SHAPE and conv(ps=0) == SHAPE and conv(ns=0) == SHAPE and conv(ld=8) == SHAPE
    assert conv(T=0) == OK and conv(cols=0) == OK
    for kw in ("tk", "cu", "kl", "qs", "bt", "out"):
        assert conv(**{kw: None}) == NULL
    assert conv(bt=P + 2) == ALIGN
    def build(tk=P, T=8, cols=16, gi=P, ui=P, ul=P, mk=P, mg=3, pad=128, G=8, cu=P):
        return lib.dsa_build_group_union_varlen(tk, 16, T, cols, 2, cu, P, P, P, 4, 64, 256, G, mg, pad,
                                                gi, ui, ul, mk, None)
    assert build(pad=100) == SHAPE and build(pad=64) == SHAPE and build(G=9) == SHAPE
    assert build(mg=0) == OK
    for kw in ("gi", "ui", "ul", "mk", "cu"):
        assert build(**{kw: None}) == NULL
    assert build(gi=P + 4) == ALIGN
    def gv(H=16, dqk=576, ns=256, mg=3, pad=128, gi=P, T=8, scale=0.1, rs=None):
        return lib.dsa_sparse_prefill_grouped_varlen(P, P, rs, ns, gi, mg, P, P, P, T, H, pad, dqk, 512, scale,
                                                     P, P, None)
    assert gv(H=24) == UNSUP and gv(dqk=448) == UNSUP and gv(scale=0.0) == UNSUP
    assert gv(dqk=512, T=0) == OK
    assert gv(ns=0) == SHAPE and gv(pad=40) == SHAPE
    assert gv(mg=0) == OK and gv(T=0) == OK and gv(gi=None) == NULL and gv(gi=P + 4) == ALIGN
    assert gv(rs=P + 2) == ALIGN
    def pv(H=16, ws=P, T=8, R_=2, cols=16, rs=None):
        return lib.dsa_sparse_prefill_pertoken_varlen(P, P, rs, 256, P, 16, T, H, cols, R_, P, P, P, P, 4, 64,
                                                      576, 512, 0.1, ws, P, P, None)
    assert pv(H=8) == UNSUP and pv(R_=0) == SHAPE and pv(T=0) == OK and pv(ws=None) == NULL
    assert pv(rs=P + 1) == ALIGN


def test_fp8_validation(lib):
    # decode pass
    def dq(kv=P, S=64, d=576, out=P):
        return lib.dsa_decode_latent_fp8(kv, S, d, out, None)
    assert dq(d=500) == UNSUP and dq(S=-1) == SHAPE and dq(S=0) == OK
    for kw in ("kv", "out"):
        assert dq(**{kw: None}) == NULL
    assert dq(kv=P + 8) == ALIGN and dq(out=P + 2) == ALIGN
    # attention over an FP8 latent: the bf16 checks first (T = 0 enqueues nothing)
    def gf(q=P, kv=P, sc=P, per_row=0, T=64, H=16, dqk=576, ws=P, pad=256):
        return lib.dsa_sparse_prefill_grouped_fp8(q, kv, sc, per_row, P, P, P, T, H, 64, pad, dqk, 512, 0.1,
                                                  ws, P, P, None)
    assert gf(H=24) == UNSUP and gf(dqk=448) == UNSUP and gf(pad=48) == SHAPE and gf(T=0) == OK
    assert gf(kv=None) == NULL and gf(sc=None) == NULL and gf(ws=None) == NULL and gf(q=None) == NULL
    assert gf(kv=P + 4) == ALIGN and gf(ws=P + 2) == ALIGN and gf(per_row=3) == SHAPE
    def pf(q=P, kv=P, sc=P, T=64, H=16, ld=32, cols=32, ws=P):
        return lib.dsa_sparse_prefill_pertoken_fp8(q, kv, sc, 1, P, ld, T, H, 64, cols, 0, 576, 512, 0.1, ws,
                                                   P, P, None)
    assert pf(H=8) == UNSUP and pf(ld=16) == SHAPE and pf(T=0) == OK
    assert pf(kv=None) == NULL and pf(ws=None) == NULL and pf(sc=P + 1) == ALIGN
    # paged decode
    def pg(kv=P, sc=P, ns=256, d=576, R_=2, kl=P, bt=P, bt_ld=4, ps=64, wsp=4, ws=P, wsc=P, wbt=P):
        return lib.dsa_decode_paged_fp8(kv, sc, 1, ns, d, R_, kl, bt, bt_ld, ps, wsp, ws, wsc, wbt, None)
    assert pg(d=192) == UNSUP and pg(ns=100) == SHAPE and pg(R_=0) == SHAPE and pg(ps=0) == SHAPE
    assert pg(wsp=-1) == SHAPE and pg(bt_ld=0) == SHAPE
    for kw in ("kv", "sc", "kl", "bt", "ws", "wsc", "wbt"):
        assert pg(**{kw: None}) == NULL
    assert pg(wbt=P + 2) == ALIGN and pg(kv=P + 4) == ALIGN and pg(wsc=P + 2) == ALIGN
