#!/usr/bin/env python3
"""Throughput of DSA sparse-MLA prefill attention on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:

  * union + membership-mask build, then grouped attention  (grouped routing)
  * per-token sparse MQA                                   (per-token routing)
  * top-k bit scatter, then masked dense MHA               (masked-MHA routing)

Default workload "glm16k": the GLM-style per-GPU share of a 16k-token prefill
chunk (T = S = 16384, H = 16, top-2048, groups of 8 tokens, 576-wide bf16
latent, scale 1/16; locality top-k, seed 2) for the two MQA routings, and the
NoPE masked-MHA layer of the same chunk (qk 256, rope 0, v 256, H = 16, scale
1/16; locality top-k, seed 3) for the masked routing.  Inputs are resident in
HBM before the timed region starts.

value = query tokens per second of the whole step (T / step time).  Per-kernel
times come from HIP events recorded on the launch stream over the timed region
(mean, median and min over the timed steps); after it, each call is also timed
"cold", right after a 1 GiB write that evicts L2 and the Infinity Cache (median
of 5, outside the timed region).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "query-tokens/s per layer (DSA sparse prefill, k=2048) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

WORKLOADS = {
    # name: (MQA config, masked-MHA config or None)
    "glm16k": ("c3_glm16k", "c4_masked_nope"),
    "glm16k_rope": ("c3_glm16k", "c6_masked_rope"),
    "glm16k_latent512": ("c7_glm16k_latent512", "c4_masked_nope"),
    # a batch of 8 requests (2048 query tokens after 14336 positions of context each) over a
    # paged cache (64-row pages in a random physical order): the two MQA routings
    "glm16k_paged": (None, None),
    "crossover": (None, None),
    # the glm16k chunk over an FP8 (E4M3, per-row scale) latent: conversion + the MQA routings
    "glm16k_fp8": (None, None),
    "glm16k_uniform": ("c3w_glm16k_uniform", None),
    "long32k": ("c5_long", None),
    "dsv32": ("c2_dsv32", "c8_masked_dsv32"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="glm16k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold (cache-flushed) timings")
    ap.add_argument("--heads", default="16,32,64,128", help="crossover: heads per GPU")
    ap.add_argument("--lengths", default="1024,2048,4096,8192,16384,32768",
                    help="crossover: chunk lengths (T = S, starting at position 0)")
    ap.add_argument("--dqk", type=int, default=576, choices=(576, 512),
                    help="crossover: latent width of the MQA routings")
    ap.add_argument("--mha", default="256,0,256", choices=("256,0,256", "192,64,256", "128,64,128"),
                    help="crossover: (qk_nope, qk_rope, v) of the MHA routings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (calibrates HBM byte counters)")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    """A plain elementwise copy of known size: reads and writes mib MiB each (counter calibration)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.add(a, 0.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_read": n * 4, "calibration_copy_bytes_written": n * 4,
                      "kernel": "elementwise add(a, 0) -> b", "dispatches": 3}), flush=True)


def algorithmic_work(case, union_len_sum, mha_case):
    """Bytes / flops each kernel must move or execute (definitions in the design notes)."""
    cfg, topk = case.cfg, case.topk
    T, S, H, cols = cfg.T, cfg.S, cfg.H, cfg.cols
    pos = cfg.q_pos_offset + np.arange(T)[:, None]
    nsel = int(((topk >= 0) & (topk < S) & (topk <= pos)).sum())
    NG = cfg.NG
    pad = -(-(cfg.G * cols) // 64) * 64
    rows_live = np.minimum(cfg.G, T - np.arange(NG) * cfg.G) * H   # live pseudo-head rows per group
    d = cfg.d_qk   # latent width: 576 (with the rope part) or 512
    w = {
        "build_union": {"bound": "hbm", "bytes": T * cols * 4 + NG * pad * 5 + NG * 4},
        "grouped_attn": {"bound": "mfma", "flops": None},   # filled below from the union lengths
        "pertoken_attn": {"bound": "hbm",
                          "bytes": nsel * 2 * d + T * H * d * 2 + T * H * 512 * 2 + T * H * 4 + T * cols * 4},
    }
    w["grouped_attn"]["flops"] = float(np.sum(union_len_sum * rows_live)) * 2 * (d + 512)
    if mha_case is not None:
        m = mha_case.cfg
        words = (m.S + 31) // 32
        causal_keys = np.minimum(m.S, m.q_pos_offset + np.arange(m.T) + 1).astype(np.float64)
        w["scatter_topk_bits"] = {"bound": "hbm", "bytes": m.T * m.cols * 4 + m.T * words * 4}
        w["masked_mha"] = {"bound": "mfma",
                           "flops": float(causal_keys.sum()) * m.H * 2 * (m.dn + m.dr + m.dv)}
    return w, nsel


KERNEL_SYMBOLS = {  # bench kernel name -> (device symbol, sources)
    "build_union": ("dsa::build_union_kernel<false>", ["union_builder.hip", "common.h"]),
    "grouped_attn": ("dsa::rows128_attn_kernel<576, false>", ["grouped_attn.hip", "common.h"]),
    "pertoken_attn": ("dsa::pertoken_sorted_kernel<576>", ["pertoken_attn.hip", "common.h"]),
    "masked_mha_routing": ("dsa::masked_mha_kernel<256, 0, 256, false>", ["masked_mha.hip", "common.h"]),
}


def source_digest(files) -> str:
    """Digest of the kernel sources' code: comments and blank lines are dropped, so an edit
    of the comments alone keeps a counter record valid."""
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(root, "mla_prefill_amd", "csrc", f)).read()
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """L2-to-memory bytes per launch from the committed rocprofv3 counter record, or None when
    there is no record for this workload or the kernel's code has changed since."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path) or kernel not in KERNEL_SYMBOLS:
        return None
    rec = json.load(open(path))
    sym, files = KERNEL_SYMBOLS[kernel]
    k = rec["kernels"].get(sym)
    if k is None:
        return None
    if source_digest(files) != k.get("source_code_sha256_16"):
        return None
    return (k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"]) * 1024.0


def cold_times(calls, names, stream, reps=5):
    """Median time of each call after a 1 GiB write that evicts L2 and the Infinity Cache."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    got = {n: [] for n in names}
    for r in range(reps):
        for n, call in zip(names, calls):
            flush.fill_(float(r))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            got[n].append(e0.elapsed_time(e1))
    del flush
    return {n: float(np.median(v)) for n, v in got.items()}


def cpu_baseline(case, mha_case, budget_s):
    """The oracle, as it stands, on whole groups sampled across the sequence."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cfg = case.cfg
    G = cfg.G
    rng = np.random.default_rng(0)
    order = rng.permutation(cfg.NG)
    done_tokens, spent = 0, 0.0
    groups = []
    for g in order:
        toks = list(range(g * G, min(cfg.T, g * G + G)))
        t0 = time.perf_counter()
        sub = case.topk[g * G:g * G + G]
        ui, ul, mk = oracle.group_union_mask(sub, cfg.S, cfg.q_pos_offset + g * G, G)
        oracle.grouped_sparse_mqa(case.q[g * G:g * G + G], case.kv, ui, ul, mk, cfg.scale)
        oracle.pertoken_sparse_mqa(case.q, case.kv, case.topk, cfg.S, cfg.q_pos_offset, cfg.scale, tokens=toks)
        if mha_case is not None:
            m = mha_case.cfg
            oracle.masked_mha(mha_case.q, mha_case.k_nope, mha_case.k_pe, mha_case.v, mha_case.topk,
                              m.S, m.q_pos_offset, m.scale, tokens=toks)
        spent += time.perf_counter() - t0
        done_tokens += len(toks)
        groups.append(int(g))
        if spent >= budget_s:
            break
    return {
        "value": done_tokens / spent,
        "unit": "query-tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(groups)} whole groups ({done_tokens} query tokens) drawn uniformly from the "
                   f"{cfg.NG} groups of the workload; every routing of the step (union/mask, grouped, "
                   f"per-token" + (", masked MHA" if mha_case is not None else "") +
                   f") on numpy float64; {spent:.1f} s"),
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); every GPU box here has one "
              "GPU and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_prefill_amd import routings
    from synth import CONFIGS, make_case

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.calibrate_copy_mib:
        calibrate_copy(a.calibrate_copy_mib)
        return

    if a.workload == "glm16k_paged":
        bench_paged(a)
        return
    if a.workload == "crossover":
        bench_crossover(a)
        return
    if a.workload == "glm16k_fp8":
        bench_fp8(a)
        return
    mqa_name, mha_name = WORKLOADS[a.workload]
    t_gen = time.perf_counter()
    case = make_case(CONFIGS[mqa_name])
    mha_case = make_case(CONFIGS[mha_name]) if mha_name else None
    cfg = case.cfg
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def dbf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    q, kv = dbf(case.q), dbf(case.kv)
    topk = torch.from_numpy(case.topk).cuda()
    G, H, T = cfg.G, cfg.H, cfg.T
    bufs = routings.alloc_union(T, G, cfg.cols)
    out_g, lse_g = routings.alloc_out(T, H, 512)
    out_p, lse_p = routings.alloc_out(T, H, 512)
    if mha_case is not None:
        m = mha_case.cfg
        mq, mk, mv = dbf(mha_case.q), dbf(mha_case.k_nope), dbf(mha_case.v)
        mkp = None if mha_case.k_pe is None else dbf(mha_case.k_pe)
        mtopk = torch.from_numpy(mha_case.topk).cuda()
        ws = torch.empty((m.T, (m.S + 31) // 32), dtype=torch.int32, device="cuda")
        out_m, lse_m = routings.alloc_out(m.T, m.H, m.dv)
    from mla_prefill_amd import _lib
    stream = torch.cuda.current_stream()

    names = ["build_union", "grouped_attn", "pertoken_attn"] + (["masked_mha_routing"] if mha_case else [])

    calls = [
        lambda: _lib.dsa_build_group_union(topk, cfg.S, cfg.q_pos_offset, G, bufs.union_idx, bufs.union_len,
                                           bufs.mask, stream=stream),
        lambda: _lib.dsa_sparse_prefill_grouped(q, kv, bufs.union_idx, bufs.union_len, bufs.mask, cfg.scale,
                                                out_g, lse_g, stream=stream),
        lambda: _lib.dsa_sparse_prefill_pertoken(q, kv, topk, cfg.q_pos_offset, cfg.scale, out_p, lse_p,
                                                 stream=stream),
    ]
    if mha_case is not None:
        calls.append(lambda: _lib.dsa_masked_mha_prefill(mq, mk, mkp, mv, mtopk, m.q_pos_offset, m.scale, ws,
                                                         out_m, lse_m, stream=stream))

    def step(ev=None):
        for i, call in enumerate(calls):
            if ev is not None:
                ev[i].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    nev = len(names) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    samples = {n: [events[s][i].elapsed_time(events[s][i + 1]) for s in range(a.steps)]
               for i, n in enumerate(names)}
    per = {n: float(np.mean(v)) for n, v in samples.items()}
    ms_step = wall * 1e3 / a.steps
    cold = {n: None for n in names} if a.no_cold else cold_times(calls, names, stream)
    if not (torch.isfinite(out_g.float()).all() and torch.isfinite(out_p.float()).all()):
        print("non-finite output", file=sys.stderr)
        sys.exit(3)

    work, nsel = algorithmic_work(case, bufs.union_len.cpu().numpy().astype(np.float64), mha_case)
    kernels = {}
    for n in names:
        key = "masked_mha" if n == "masked_mha_routing" else n
        wk = work[key]
        ms = per[n]
        if wk["bound"] == "hbm":
            ach = wk["bytes"] / (ms * 1e-3) / 1e9
            kernels[n] = {"ms": ms, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": ach / HBM_PEAK_GBS, "algorithmic": wk["bytes"]}
        else:
            ach = wk["flops"] / (ms * 1e-3) / 1e12
            kernels[n] = {"ms": ms, "bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFS,
                          "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFS, "algorithmic": wk["flops"]}
        kernels[n].update({"median_ms": float(np.median(samples[n])), "min_ms": float(np.min(samples[n])),
                           "cold_ms": cold[n]})
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    d = kernels[dom]
    traffic = measured_traffic(dom, a.workload)
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": round(d["achieved"], 2), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["frac"], 4),
                "traffic": None if traffic is None else round(traffic)}
    routing_tps = {
        "grouped (union build + attention)": T / ((per["build_union"] + per["grouped_attn"]) * 1e-3),
        "per-token": T / (per["pertoken_attn"] * 1e-3),
    }
    if mha_case is not None:
        routing_tps["masked MHA (bit scatter + attention)"] = mha_case.cfg.T / (per["masked_mha_routing"] * 1e-3)

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(case, mha_case, a.cpu_seconds)

    config = {"workload": a.workload, "mqa": mqa_name, "d_qk": cfg.d_qk, "T": cfg.T, "S": cfg.S, "H": cfg.H,
              "k": cfg.k,
              "cols": cfg.cols, "G": cfg.G, "q_pos_offset": cfg.q_pos_offset,
              "selected_rows": nsel}
    if mha_case is not None:
        config["masked_mha"] = {"config": mha_name, "dn": m.dn, "dr": m.dr, "dv": m.dv, "H": m.H}
    line = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "routing_query_tokens_per_s": {k: round(v, 1) for k, v in routing_tps.items()},
    }
    print(json.dumps(line), flush=True)


PAGED = dict(seed=6, q_lens=[2048] * 8, ctx_lens=[14336] * 8, H=16, k=2048, cols=2048, page_size=64,
             G=8, mode="locality", spare_pages=64)


def cpu_baseline_paged(case, budget_s):
    """The oracle on whole groups of the batch sampled across its requests."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    groups = oracle.varlen_groups(case.cu_seqlens, case.G)
    args = (case.cu_seqlens, case.kv_lens, case.q_pos_start, case.block_table, case.page_size)
    rng = np.random.default_rng(0)
    done, spent, n = 0, 0.0, 0
    for gi in rng.permutation(len(groups)):
        t0, cnt = groups[gi]
        toks = list(range(t0, t0 + cnt))
        start = time.perf_counter()
        r = int(np.searchsorted(case.cu_seqlens, t0, side="right") - 1)
        sub_cu = np.array([0, cnt])
        sub = (sub_cu, case.kv_lens[r:r + 1], case.q_pos_start[r:r + 1] + (t0 - case.cu_seqlens[r]),
               case.block_table[r:r + 1], case.page_size)
        info, ui, ul, mk = oracle.group_union_mask_varlen(case.topk[t0:t0 + cnt], *sub, case.num_slots,
                                                          case.G, 1)
        oracle.grouped_sparse_mqa_varlen(case.q[t0:t0 + cnt], case.kv_cache, info, ui, ul, mk, case.scale)
        oracle.pertoken_sparse_mqa_varlen(case.q, case.kv_cache, case.topk, *args, case.scale, tokens=toks)
        spent += time.perf_counter() - start
        done += cnt
        n += 1
        if spent >= budget_s:
            break
    return {"value": done / spent, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{n} whole groups ({done} query tokens) drawn uniformly from the {len(groups)} groups "
                       f"of the batch; union/mask, grouped and per-token on numpy float64; {spent:.1f} s")}


def bench_paged(a):
    """The two MQA routings on a batch of requests over a paged cache."""
    import torch
    from mla_prefill_amd import _lib, routings
    from synth import make_varlen_case

    t_gen = time.perf_counter()
    c = make_varlen_case(**PAGED)
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def dbf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    def di(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()

    q, kv, tk = dbf(c.q), dbf(c.kv_cache), di(c.topk)
    batch = (di(c.cu_seqlens), di(c.kv_lens), di(c.q_pos_start), di(c.block_table), c.page_size)
    T, H = q.shape[0], q.shape[1]
    mg = c.max_groups()
    bufs = routings.alloc_union_varlen(mg, c.G, c.topk.shape[1])
    out_g, lse_g = routings.alloc_out(T, H, 512)
    out_p, lse_p = routings.alloc_out(T, H, 512)
    ws = torch.empty_like(tk)
    stream = torch.cuda.current_stream()
    names = ["build_union", "grouped_attn", "pertoken_attn"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        _lib.dsa_build_group_union_varlen(tk, batch, c.num_slots, c.G, bufs.group_info, bufs.union_idx,
                                          bufs.union_len, bufs.mask, stream=stream)
        mark(1)
        _lib.dsa_sparse_prefill_grouped_varlen(q, kv, bufs.group_info, bufs.union_idx, bufs.union_len,
                                               bufs.mask, c.scale, out_g, lse_g, stream=stream)
        mark(2)
        _lib.dsa_sparse_prefill_pertoken_varlen(q, kv, tk, batch, c.scale, ws, out_p, lse_p, stream=stream)
        mark(3)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(a.steps):
        step(events[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: float(np.mean([events[s_][i].elapsed_time(events[s_][i + 1]) for s_ in range(a.steps)]))
           for i, n in enumerate(names)}
    ms_step = wall * 1e3 / a.steps
    if not (torch.isfinite(out_g.float()).all() and torch.isfinite(out_p.float()).all()):
        print("non-finite output", file=sys.stderr)
        sys.exit(3)

    # algorithmic work: union over the groups' rows, selected rows of every token
    info = bufs.group_info.cpu().numpy()
    ul = bufs.union_len.cpu().numpy().astype(np.float64)
    nsel = int((ws.cpu().numpy() >= 0).sum())
    cols = c.topk.shape[1]
    pad = bufs.union_idx.shape[1]
    work = {
        "build_union": ("hbm", T * cols * 4 + mg * pad * 5 + mg * 12),
        "grouped_attn": ("mfma", float(np.sum(ul * info[:, 1] * H)) * 2 * (576 + 512)),
        "pertoken_attn": ("hbm", nsel * 1152 + T * H * 576 * 2 + T * H * 512 * 2 + T * H * 4 + T * cols * 8),
    }
    kernels = {}
    for n in names:
        bound, amount = work[n]
        ms = per[n]
        if bound == "hbm":
            ach = amount / (ms * 1e-3) / 1e9
            kernels[n] = {"ms": ms, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": ach / HBM_PEAK_GBS, "algorithmic": amount}
        else:
            ach = amount / (ms * 1e-3) / 1e12
            kernels[n] = {"ms": ms, "bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFS,
                          "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFS, "algorithmic": amount}
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    d = kernels[dom]
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": round(d["achieved"], 2), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["frac"], 4), "traffic": None}
    cpu = None if a.no_cpu else cpu_baseline_paged(c, a.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "glm16k_paged", "requests": len(PAGED["q_lens"]), "q_len": PAGED["q_lens"][0],
                   "ctx": PAGED["ctx_lens"][0], "H": H, "k": PAGED["k"], "cols": cols, "G": c.G,
                   "page_size": c.page_size, "num_slots": c.num_slots, "groups": mg, "selected_rows": nsel},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "routing_query_tokens_per_s": {
            "grouped (union build + attention)": round(T / ((per["build_union"] + per["grouped_attn"]) * 1e-3), 1),
            "per-token (index conversion + attention)": round(T / (per["pertoken_attn"] * 1e-3), 1)},
    }
    print(json.dumps(line), flush=True)


def bench_fp8(a):
    """The glm16k chunk (c3 shapes and top-k) over an FP8 latent: the conversion pass into the
    bf16 workspace, then union + grouped attention and per-token attention on it."""
    import torch
    from mla_prefill_amd import _lib, routings
    from synth import CONFIGS, make_case, normal_fp8

    cfg = CONFIGS["c3_glm16k"]
    t_gen = time.perf_counter()
    case = make_case(cfg)
    codes, kscale = normal_fp8(np.random.default_rng(9), cfg.S, cfg.d_qk, per_row=True)
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    q = torch.from_numpy(case.q.view(np.int16)).cuda().view(torch.bfloat16)
    topk = torch.from_numpy(case.topk).cuda()
    kv8 = torch.from_numpy(codes).cuda()
    ksc = torch.from_numpy(kscale).cuda()
    T, H, G, S = cfg.T, cfg.H, cfg.G, cfg.S
    ws = routings.alloc_latent_ws(S, cfg.d_qk)
    bufs = routings.alloc_union(T, G, cfg.cols)
    out_g, lse_g = routings.alloc_out(T, H, 512)
    out_p, lse_p = routings.alloc_out(T, H, 512)
    stream = torch.cuda.current_stream()
    names = ["dequant_fp8", "build_union", "grouped_attn", "pertoken_attn"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        _lib.dsa_dequant_latent_fp8(kv8, ksc, ws, stream=stream)
        mark(1)
        _lib.dsa_build_group_union(topk, S, 0, G, bufs.union_idx, bufs.union_len, bufs.mask, stream=stream)
        mark(2)
        _lib.dsa_sparse_prefill_grouped(q, ws, bufs.union_idx, bufs.union_len, bufs.mask, cfg.scale, out_g,
                                        lse_g, stream=stream)
        mark(3)
        _lib.dsa_sparse_prefill_pertoken(q, ws, topk, 0, cfg.scale, out_p, lse_p, stream=stream)
        mark(4)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for s_ in range(a.steps):
        step(events[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: float(np.mean([events[s_][i].elapsed_time(events[s_][i + 1]) for s_ in range(a.steps)]))
           for i, n in enumerate(names)}
    ms_step = wall * 1e3 / a.steps
    work, nsel = algorithmic_work(case, bufs.union_len.cpu().numpy().astype(np.float64), None)
    work["dequant_fp8"] = {"bound": "hbm", "bytes": S * cfg.d_qk * 3 + S * 4}
    kernels = {}
    for n in names:
        wk, ms = work[n], per[n]
        if wk["bound"] == "hbm":
            ach = wk["bytes"] / (ms * 1e-3) / 1e9
            kernels[n] = {"ms": ms, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": ach / HBM_PEAK_GBS, "algorithmic": wk["bytes"]}
        else:
            ach = wk["flops"] / (ms * 1e-3) / 1e12
            kernels[n] = {"ms": ms, "bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFS,
                          "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFS, "algorithmic": wk["flops"]}
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    d = kernels[dom]
    line = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8 latent, bf16 compute", "data": "synthetic",
        "config": {"workload": "glm16k_fp8", "T": T, "S": S, "H": H, "k": cfg.k, "G": G, "d_qk": cfg.d_qk,
                   "fp8": "E4M3, per-row float32 scale", "selected_rows": nsel},
        "roofline": {"kernel": dom, "bound": d["bound"], "achieved": round(d["achieved"], 2), "peak": d["peak"],
                     "unit": d["unit"], "frac": round(d["frac"], 4), "traffic": None},
        "cpu_baseline": None,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
    }
    print(json.dumps(line), flush=True)



def bench_crossover(a):
    """Every routing of the same chunk across lengths and head counts (the routing decision).

    For each chunk length L (T = S = L from position 0, top-2048 with 8-token locality, seed
    10 + L) and each head count H (G = 128 / H): the grouped routing (union build + attention)
    and the per-token routing over the latent (576 wide, or --dqk 512), the masked routing (bit scatter +
    attention) over per-head K/V (--mha: NoPE (256, 0, 256) by default), and for L <= k the
    dense shortcut.
    Values are N(0, 1) bf16 drawn on the device from a seeded generator (timing only: parity of
    every kernel is covered by the tests).  Median over --steps timed calls after --warmup.
    One JSON line per (H, L), then a summary line with the fastest routing per point.
    """
    import torch
    from mla_prefill_amd import _lib, routings
    from synth.gen import topk_locality

    heads = [int(x) for x in a.heads.split(",")]
    lengths = [int(x) for x in a.lengths.split(",")]
    k = cols = 2048
    scale = 1.0 / 16.0
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")

    def randn_bf16(shape, seed):
        gen.manual_seed(seed)
        return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        ms = []
        for _ in range(a.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    summary = {}
    for L in lengths:
        rng = np.random.default_rng(10 + L)
        topk = torch.from_numpy(topk_locality(rng, L, L, k, cols, 8)).cuda()
        for H in heads:
            G = 128 // H
            seed = 1000 * L + H
            q, kv = randn_bf16((L, H, a.dqk), seed), randn_bf16((L, a.dqk), seed + 1)
            bufs = routings.alloc_union(L, G, cols)
            og, lg = routings.alloc_out(L, H, 512)
            op, lp = routings.alloc_out(L, H, 512)

            def grouped():
                _lib.dsa_build_group_union(topk, L, 0, G, bufs.union_idx, bufs.union_len, bufs.mask,
                                           stream=stream)
                _lib.dsa_sparse_prefill_grouped(q, kv, bufs.union_idx, bufs.union_len, bufs.mask, scale,
                                                og, lg, stream=stream)

            def pertoken():
                _lib.dsa_sparse_prefill_pertoken(q, kv, topk, 0, scale, op, lp, stream=stream)

            ms = {"grouped": timed(grouped), "per-token": timed(pertoken)}
            del q, kv, bufs, og, lg, op, lp
            dn, dr, dv = (int(x) for x in a.mha.split(","))
            mq = randn_bf16((L, H, dn + dr), seed + 2)
            mk = randn_bf16((L, H, dn), seed + 3)
            mv = randn_bf16((L, H, dv), seed + 4)
            mkp = randn_bf16((L, dr), seed + 5) if dr else None
            ws = torch.empty((L, (L + 31) // 32), dtype=torch.int32, device="cuda")
            om, lm = routings.alloc_out(L, H, dv)

            def masked():
                _lib.dsa_masked_mha_prefill(mq, mk, mkp, mv, topk, 0, scale, ws, om, lm, stream=stream)

            def dense():
                _lib.dsa_dense_mha_prefill(mq, mk, mkp, mv, 0, scale, om, lm, stream=stream)

            ms["masked"] = timed(masked)
            if L <= k:
                ms["dense"] = timed(dense)
            del mq, mk, mv, mkp, ws, om, lm
            torch.cuda.empty_cache()
            best = min(ms, key=ms.get)
            summary[f"H{H}_L{L}"] = best
            print(json.dumps({"workload": "crossover", "H": H, "G": G, "L": L, "k": k, "d_qk": a.dqk,
                              "mha": a.mha,
                              "ms": {r: round(v, 4) for r, v in ms.items()}, "fastest": best,
                              "query_tokens_per_s": {r: round(L / (v * 1e-3), 1) for r, v in ms.items()}}),
                  flush=True)
    print(json.dumps({"workload": "crossover", "fastest": summary}), flush=True)


if __name__ == "__main__":
    main()
