#!/usr/bin/env python3
"""Throughput of DSA sparse-MLA prefill attention on one MI355X.

One step is one layer of sparse prefill attention over one chunk of synthetic
input, computed by the routing the library itself picks for the chunk.  The
choice has two stages: ``dsa_select_routing`` weighs the MHA forms against the
sparse MQA forms from the chunk's lengths (host side), and where it picks the
grouped form (H = 16, 32, 64) the step is one ``dsa_sparse_prefill_auto`` call:
union + membership-mask build, then one workgroup that compares the union's
32-slot tiles with the per-token cost and lets only the cheaper of grouped and
per-token attention run (the other returns at once).  The default workload
"glm16k" is the GLM-style per-GPU share of a 16k-token prefill chunk
(T = S = 16384, H = 16, top-2048, groups of 8 tokens, 576-wide bf16 latent,
scale 1/16; locality top-k, seed 2), where the grouped form runs, and

    value = query tokens per second of one layer (T / step time).

Inputs are resident in HBM before the timed region starts.  Per-kernel times
come from HIP events recorded on the launch stream around each kernel's own
calls (mean, median and min over --steps calls after --warmup, the form the
union-size routing ran timed kernel by kernel, since one ``auto`` call enqueues
all of them); after the timed region each kernel is also timed "cold", right
after a 1 GiB write that evicts L2 and the Infinity Cache.

Extra keys of the same JSON line (not part of ``value``):

* ``routings``: the other routings of the same layer, each timed alone over
  --steps calls: per-token sparse MQA on the same inputs, and the masked dense
  MHA (top-k bit scatter + attention) of the NoPE (256, 0, 256) layer of the
  same chunk (c4 shapes, seed 3);
* ``configs``: the other single-GPU configurations -- the long prompt (32k KV,
  the last 21504 positions as queries, 2176-column top-k buffer), the
  worst-case uniform top-k over the 16k chunk (unions up to 10.8k rows, where
  the union-size routing runs per-token), and the DeepSeek-V3.2-style layer
  (H = 128, T = S = 4096) -- with the routing the library picks for each, every
  routing timed with its roofline fraction, and the ``auto`` call's own time,
  the form it ran and its overhead over that form.

Roofline bounds (algorithmic work per launch over its mean launch time):
grouped, per-token and masked attention against dense bf16 MFMA
(2.5 PFLOP/s): they are contractions whose operands come from L2 (the
per-token gather is served mostly by L2, see ``traffic``); the union build and
the bit scatter against HBM (8 TB/s).

``cpu_baseline``: the oracle (numpy float64), as it stands, computing the
chosen routing (union/mask + grouped attention) on whole groups sampled across
the chunk, sharded over worker processes (one BLAS thread each), on the host
cores this process may use (at most 16).

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
CPU_WORKERS_MAX = 16           # the host CPU share of one GPU

# workload name -> (MQA config, MHA config of the same layer or None, extra configs)
WORKLOADS = {
    "glm16k": ("c3_glm16k", "c4_masked_nope", ("c5_long", "c3w_glm16k_uniform", "c2_dsv32")),
    "glm16k_rope": ("c3_glm16k", "c6_masked_rope", ()),
    "glm16k_latent512": ("c7_glm16k_latent512", "c4_masked_nope", ()),
    "glm16k_uniform": ("c3w_glm16k_uniform", "c4_masked_nope", ()),
    "long32k": ("c5_long", None, ()),
    "dsv32": ("c2_dsv32", "c8_masked_dsv32", ()),
    # a batch of 8 requests (2048 query tokens after 14336 positions of context each) over a
    # paged cache (64-row pages in a random physical order): the two MQA routings
    "glm16k_paged": (None, None, ()),
    "crossover": (None, None, ()),
    # the glm16k chunk over an FP8 (E4M3, per-row scale) latent: decode + the MQA routings
    "glm16k_fp8": (None, None, ()),
}
# the MHA layer each MQA configuration can also run as (value width of its geometry)
MHA_OF = {"c2_dsv32": "c8_masked_dsv32", "c3_glm16k": "c4_masked_nope", "c3w_glm16k_uniform": "c4_masked_nope",
          "c5_long": None, "c7_glm16k_latent512": "c4_masked_nope"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="glm16k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold (cache-flushed) timings")
    ap.add_argument("--no-extra", action="store_true", help="skip the other routings and configurations")
    ap.add_argument("--heads", default="16,32,64,128", help="crossover: heads per GPU")
    ap.add_argument("--lengths", default="1024,2048,4096,8192,16384,32768",
                    help="crossover: chunk lengths (T = S, starting at position 0)")
    ap.add_argument("--dqk", type=int, default=576, choices=(576, 512),
                    help="crossover: latent width of the MQA routings")
    ap.add_argument("--mha", default="256,0,256", choices=("256,0,256", "192,64,256", "128,64,128"),
                    help="crossover: (qk_nope, qk_rope, v) of the MHA routings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="wall-time budget of the oracle sample")
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


# ---------------------------------------------------------------------------
# algorithmic work per launch (definitions in the design notes)
# ---------------------------------------------------------------------------

def selected_rows(cfg, topk) -> int:
    pos = cfg.q_pos_offset + np.arange(cfg.T)[:, None]
    return int(((topk >= 0) & (topk < cfg.S) & (topk <= pos)).sum())


def mqa_work(cfg, topk, union_len):
    """Work of the MQA kernels of one configuration: bytes for the union build (HBM), flops
    for the attention kernels (bf16 MFMA), and the per-token kernel's gathered bytes."""
    T, S, H, cols, G = cfg.T, cfg.S, cfg.H, cfg.cols, cfg.G
    NG = cfg.NG
    d = cfg.d_qk
    nsel = selected_rows(cfg, topk)
    rows_live = np.minimum(G, T - np.arange(NG) * G) * H   # live pseudo-head rows per group
    return {
        # the top-k rows read, the union entries and their mask bytes written, union_len
        "build_union": ("hbm", T * cols * 4 + int(np.sum(union_len)) * 5 + NG * 4),
        "grouped_attn": ("mfma", float(np.sum(np.asarray(union_len, np.float64) * rows_live)) * 2 * (d + 512)),
        "pertoken_attn": ("mfma", float(nsel) * H * 2 * (d + 512)),
        "pertoken_gather_bytes": nsel * 2 * d,
    }, nsel


def mha_work(m):
    words = (m.S + 31) // 32
    causal_keys = np.minimum(m.S, m.q_pos_offset + np.arange(m.T) + 1).astype(np.float64)
    return {
        "scatter_topk_bits": ("hbm", m.T * m.cols * 4 + m.T * words * 4),
        "masked_mha": ("mfma", float(causal_keys.sum()) * m.H * 2 * (m.dn + m.dr + m.dv)),
    }


def kernel_record(samples, bound, amount, cold=None):
    ms = float(np.mean(samples))
    if bound == "hbm":
        ach = amount / (ms * 1e-3) / 1e9
        rec = {"ms": ms, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": ach / HBM_PEAK_GBS, "algorithmic": amount}
    else:
        ach = amount / (ms * 1e-3) / 1e12
        rec = {"ms": ms, "bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
               "frac": ach / MFMA_BF16_PEAK_TFS, "algorithmic": amount}
    rec.update({"median_ms": float(np.median(samples)), "min_ms": float(np.min(samples))})
    if cold is not None:
        rec["cold_ms"] = cold
    return rec


def rounded(d):
    if isinstance(d, dict):
        return {k: rounded(v) for k, v in d.items()}
    if isinstance(d, float):
        return round(d, 4) if abs(d) < 1e6 else round(d, 1)
    return d


KERNEL_SYMBOLS = {  # bench kernel name -> (device symbol, sources)
    "build_union": ("dsa::build_union_kernel<false>", ["union_builder.hip", "common.h"]),
    "grouped_attn": ("dsa::rows128_attn_kernel<576, false, false, true>", ["grouped_attn.hip", "common.h"]),
    "pertoken_attn": ("dsa::pertoken_sorted_kernel<576, false>", ["pertoken_attn.hip", "common.h"]),
    "masked_mha": ("dsa::masked_mha_kernel<256, 0, 256, false>", ["masked_mha.hip", "common.h"]),
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


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def time_calls(calls, stream, steps, warmup):
    """Run `calls` (a list of (name, fn), one step) warmup times, then time `steps` steps with
    HIP events on the launch stream between consecutive calls, bracketed by device
    synchronizations.  Returns ({name: [ms per step]}, wall ms per step)."""
    import torch
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for i, (_, fn) in enumerate(calls):
            ev[s][i].record(stream)
            fn()
        ev[s][len(calls)].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    samples = {n: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)] for i, (n, _) in enumerate(calls)}
    return samples, wall * 1e3 / steps


def cold_times(calls, stream, reps=5):
    """Median time of each call after a 1 GiB write that evicts L2 and the Infinity Cache."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    got = {n: [] for n, _ in calls}
    for r in range(reps):
        for n, fn in calls:
            flush.fill_(float(r))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            got[n].append(e0.elapsed_time(e1))
    del flush
    return {n: float(np.median(v)) for n, v in got.items()}


# ---------------------------------------------------------------------------
# the oracle on the host cores
# ---------------------------------------------------------------------------

_CPU = {}


def _cpu_init(kv, S, q_pos_offset, scale, G):
    _CPU.update(kv=kv, S=S, P0=q_pos_offset, scale=scale, G=G)


def _cpu_group(task):
    """Oracle of the grouped routing for one group: union/mask, then grouped attention."""
    import oracle
    g, q_rows, topk_rows = task
    G = _CPU["G"]
    t0 = time.perf_counter()
    ui, ul, mk = oracle.group_union_mask(topk_rows, _CPU["S"], _CPU["P0"] + g * G, G)
    oracle.grouped_sparse_mqa(q_rows, _CPU["kv"], ui, ul, mk, _CPU["scale"])
    return topk_rows.shape[0], time.perf_counter() - t0


def _cpu_noop(_):
    return os.getpid()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s):
    """The oracle of the chosen (grouped) routing on whole groups sampled uniformly across the
    chunk, sharded over worker processes.  Runs before this process touches the GPU; the
    workers import numpy and the oracle only."""
    import multiprocessing as mp
    import oracle
    cfg = case.cfg
    G = cfg.G
    workers = max(1, min(CPU_WORKERS_MAX, len(os.sched_getaffinity(0))))
    order = np.random.default_rng(0).permutation(cfg.NG)

    def task(g):
        return (int(g), case.q[g * G:g * G + G], case.topk[g * G:g * G + G])

    # one group in this process sizes the sample to the budget
    t0 = time.perf_counter()
    sub = case.topk[order[0] * G:order[0] * G + G]
    ui, ul, mk = oracle.group_union_mask(sub, cfg.S, cfg.q_pos_offset + order[0] * G, G)
    oracle.grouped_sparse_mqa(case.q[order[0] * G:order[0] * G + G], case.kv, ui, ul, mk, cfg.scale)
    per_group = max(time.perf_counter() - t0, 1e-3)
    n = int(min(cfg.NG, max(workers, budget_s * workers / per_group)))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_cpu_init, initargs=(case.kv, cfg.S, cfg.q_pos_offset, cfg.scale, G)) as pool:
            pool.map(_cpu_noop, range(4 * workers))           # every worker up and initialized
            t0 = time.perf_counter()
            res = pool.map(_cpu_group, (task(g) for g in order[:n]), chunksize=1)
            wall = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    tokens = sum(r[0] for r in res)
    busy = sum(r[1] for r in res)
    return {
        "value": tokens / wall,
        "unit": "query-tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{n} of the {cfg.NG} groups ({tokens} query tokens), drawn uniformly across the chunk; "
                   f"union/mask + grouped attention (the chosen routing) on numpy float64, sharded over "
                   f"{workers} worker processes with one BLAS thread each; {wall:.1f} s wall, "
                   f"{busy:.1f} s of worker time; CPU: {cpu_model()}"),
    }


# ---------------------------------------------------------------------------
# one configuration on the GPU
# ---------------------------------------------------------------------------

def _dbf(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def mqa_routings(case, stream):
    """Device inputs and the calls of the two MQA routings of one configuration:
    {"grouped": [(kernel, fn), ...], "per-token": [...]}, plus the union buffers."""
    import torch
    from mla_prefill_amd import _lib, routings
    cfg = case.cfg
    q, kv = _dbf(case.q), _dbf(case.kv)
    topk = torch.from_numpy(case.topk).cuda()
    bufs = routings.alloc_union(cfg.T, cfg.G, cfg.cols)
    out_g, lse_g = routings.alloc_out(cfg.T, cfg.H, 512)
    out_p, lse_p = routings.alloc_out(cfg.T, cfg.H, 512)
    calls = {}
    if cfg.H < 128:
        calls["grouped"] = [
            ("build_union", lambda: _lib.dsa_build_group_union(topk, cfg.S, cfg.q_pos_offset, cfg.G, bufs.union_idx,
                                                               bufs.union_len, bufs.mask, stream=stream)),
            ("grouped_attn", lambda: _lib.dsa_sparse_prefill_grouped(q, kv, bufs.union_idx, bufs.union_len,
                                                                     bufs.mask, cfg.scale, out_g, lse_g,
                                                                     stream=stream)),
        ]
    calls["per-token"] = [
        ("pertoken_attn", lambda: _lib.dsa_sparse_prefill_pertoken(q, kv, topk, cfg.q_pos_offset, cfg.scale, out_p,
                                                                   lse_p, stream=stream)),
    ]
    keep = (q, kv, topk, bufs, out_g, lse_g, out_p, lse_p)
    route = None
    if cfg.H in (16, 32, 64):
        # the library's union-size routing: union build, the decision, and the chosen form, in one call
        bufs_a = routings.alloc_union(cfg.T, cfg.G, cfg.cols)
        out_a, lse_a = routings.alloc_out(cfg.T, cfg.H, 512)
        route = torch.zeros(4, dtype=torch.int32, device="cuda")
        calls["auto"] = [
            ("auto", lambda: _lib.dsa_sparse_prefill_auto(q, kv, topk, cfg.q_pos_offset, cfg.scale, bufs_a.union_idx,
                                                          bufs_a.union_len, bufs_a.mask, route, out_a, lse_a,
                                                          stream=stream)),
        ]
        keep = keep + (bufs_a, out_a, lse_a, route)
    return calls, bufs, keep, route


def auto_summary(samples, cfg_T, route, routings):
    """The union-size routing of one configuration: its time per call and the form it ran."""
    r = route.cpu().numpy()
    ran = "per-token" if r[0] else "grouped"
    ms = float(np.mean(samples))
    return {"ms": ms, "median_ms": float(np.median(samples)), "min_ms": float(np.min(samples)),
            "query_tokens_per_s": cfg_T / (ms * 1e-3), "ran": ran, "union_tiles": int(r[2]),
            "overhead_ms": ms - routings[ran]["ms"]}


def mha_routing(mcase, stream):
    import torch
    from mla_prefill_amd import _lib, routings
    m = mcase.cfg
    mq, mk, mv = _dbf(mcase.q), _dbf(mcase.k_nope), _dbf(mcase.v)
    mkp = None if mcase.k_pe is None else _dbf(mcase.k_pe)
    mtopk = torch.from_numpy(mcase.topk).cuda()
    ws = torch.empty((m.T, (m.S + 31) // 32), dtype=torch.int32, device="cuda")
    out_m, lse_m = routings.alloc_out(m.T, m.H, m.dv)
    calls = [("masked_mha", lambda: _lib.dsa_masked_mha_prefill(mq, mk, mkp, mv, mtopk, m.q_pos_offset, m.scale, ws,
                                                                out_m, lse_m, stream=stream))]
    return calls, (mq, mk, mv, mkp, mtopk, ws, out_m, lse_m)


def routing_summary(cfg_T, kernels):
    ms = sum(k["ms"] for k in kernels.values())
    return {"ms": ms, "query_tokens_per_s": cfg_T / (ms * 1e-3), "kernels": kernels}


def measure_config(name, a, stream, want_cold=False):
    """Every routing of one configuration, the routing the library picks for it, and the
    per-kernel records.  Returns (summary dict, chosen routing name, calls of the chosen
    routing, kept device tensors)."""
    import torch
    from mla_prefill_amd import _lib
    from synth import CONFIGS, make_case
    t_gen = time.perf_counter()
    case = make_case(CONFIGS[name])
    mname = MHA_OF.get(name)
    mcase = make_case(CONFIGS[mname]) if mname else None
    cfg = case.cfg
    print(f"# [{name}] inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    mha_dv = mcase.cfg.dv if mcase is not None else 0
    chosen = _lib.dsa_select_routing(cfg.T, cfg.S, cfg.q_pos_offset, cfg.H, cfg.k, mha_dv)
    calls, bufs, keep, route = mqa_routings(case, stream)
    if chosen == "grouped" and "auto" in calls:
        chosen = "auto"  # the grouped form where the union is compact, else per-token (decided on the device)
    if mcase is not None:
        mcalls, mkeep = mha_routing(mcase, stream)
        calls["masked"] = mcalls
        keep = keep + mkeep
    samples = {}
    for r, cl in calls.items():
        s, _ = time_calls(cl, stream, a.steps, a.warmup)
        samples.update(s)
    torch.cuda.synchronize()
    union_len = bufs.union_len.cpu().numpy() if "grouped" in calls else None
    work, nsel = mqa_work(cfg, case.topk, union_len if union_len is not None else np.zeros(cfg.NG))
    if mcase is not None:
        work.update(mha_work(mcase.cfg))
    cold = (cold_times([c for r, cl in calls.items() if r != "auto" for c in cl], stream)
            if want_cold and not a.no_cold else {})
    routings = {}
    for r, cl in calls.items():
        if r == "auto":
            continue
        ks = {}
        for kname, _ in cl:
            bound, amount = work[kname]
            ks[kname] = kernel_record(samples[kname], bound, amount, cold.get(kname))
            if kname == "pertoken_attn":
                # the gathered rows per second: mostly served by L2 (see `traffic`), not an HBM figure
                ks[kname]["gathered_gbs"] = work["pertoken_gather_bytes"] / (ks[kname]["ms"] * 1e-3) / 1e9
        routings[r] = routing_summary(mcase.cfg.T if r == "masked" else cfg.T, ks)
    if "auto" in calls:
        routings["auto"] = auto_summary(samples["auto"], cfg.T, route, routings)
    summary = {
        "config": {"name": name, "T": cfg.T, "S": cfg.S, "H": cfg.H, "k": cfg.k, "cols": cfg.cols, "G": cfg.G,
                   "q_pos_offset": cfg.q_pos_offset, "d_qk": cfg.d_qk, "topk": cfg.topk_mode,
                   "selected_rows": nsel,
                   "mha": None if mcase is None else {"config": mname, "dn": mcase.cfg.dn, "dr": mcase.cfg.dr,
                                                       "dv": mcase.cfg.dv, "H": mcase.cfg.H}},
        "chosen_routing": chosen,
        "routings": routings,
    }
    if union_len is not None:
        summary["config"]["union_len_mean"] = float(np.mean(union_len))
        summary["config"]["union_len_max"] = int(np.max(union_len))
    return summary, chosen, calls, keep, case, route


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); every GPU box here has one "
              "GPU and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if a.workload in ("glm16k_paged", "crossover", "glm16k_fp8") or a.calibrate_copy_mib:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        if a.calibrate_copy_mib:
            calibrate_copy(a.calibrate_copy_mib)
        elif a.workload == "glm16k_paged":
            bench_paged(a)
        elif a.workload == "crossover":
            bench_crossover(a)
        else:
            bench_fp8(a)
        return

    from synth import CONFIGS, make_case
    mqa_name, _, extra = WORKLOADS[a.workload]
    # the oracle runs first, on the host cores, before this process initializes the GPU
    cpu = None
    if not a.no_cpu:
        t_gen = time.perf_counter()
        c0 = make_case(CONFIGS[mqa_name])
        print(f"# [{mqa_name}] oracle inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(c0, a.cpu_seconds)
        del c0
        print(f"# cpu_baseline: {cpu['value']:.1f} query-tokens/s on {cpu['cores']} processes", file=sys.stderr,
              flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    stream = torch.cuda.current_stream()

    summary, chosen, calls, keep, case, route = measure_config(mqa_name, a, stream, want_cold=True)
    cfg = case.cfg
    step_calls = calls[chosen]
    # the timed steps: one layer by the chosen routing
    samples, ms_step = time_calls(step_calls, stream, a.steps, a.warmup)
    kernels = {}
    if chosen == "auto":
        # one call enqueues every kernel of the step: its per-kernel records are those of the
        # form it ran, timed kernel by kernel above
        ran = summary["routings"]["auto"]["ran"]
        kernels = {k: dict(v) for k, v in summary["routings"][ran]["kernels"].items()}
        kernels["auto"] = {"ms": float(np.mean(samples["auto"])), "median_ms": float(np.median(samples["auto"])),
                           "min_ms": float(np.min(samples["auto"])), "ran": ran}
    else:
        step_routing = summary["routings"][chosen]
        for kname, _ in step_calls:
            rec = dict(step_routing["kernels"][kname])
            fresh = kernel_record(samples[kname], rec["bound"], rec["algorithmic"], rec.get("cold_ms"))
            if "gathered_gbs" in rec:
                fresh["gathered_gbs"] = rec["gathered_gbs"] * rec["ms"] / fresh["ms"]
            kernels[kname] = fresh
    del keep
    torch.cuda.empty_cache()
    dom = max((k for k in kernels if k != "auto"), key=lambda k: kernels[k]["ms"])
    d = kernels[dom]
    traffic = measured_traffic(dom, a.workload)
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": round(d["achieved"], 2), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["frac"], 4),
                "traffic": None if traffic is None else round(traffic)}

    others = {}
    if not a.no_extra:
        for name in extra:
            s, *_rest = measure_config(name, a, stream)
            others[name] = s
            del _rest
            torch.cuda.empty_cache()

    config = {"workload": a.workload, **{k: v for k, v in summary["config"].items() if k != "name"},
              "mqa_config": mqa_name, "routing": chosen}
    line = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_step * 1e-3), 1),
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
        "kernels": rounded(kernels),
        "routings": rounded(summary["routings"]),
        "configs": rounded(others),
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
        "pertoken_attn": ("mfma", float(nsel) * H * 2 * (576 + 512)),
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
    # the step is the grouped routing (union build + attention): its dominant kernel
    dom = max(("build_union", "grouped_attn"), key=lambda k: kernels[k]["ms"])
    d = kernels[dom]
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": round(d["achieved"], 2), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["frac"], 4), "traffic": None}
    cpu = None if a.no_cpu else cpu_baseline_paged(c, a.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(T / ((per["build_union"] + per["grouped_attn"]) * 1e-3), 1),
        "unit": "query-tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(per["build_union"] + per["grouped_attn"], 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "glm16k_paged", "routing": "grouped", "requests": len(PAGED["q_lens"]), "q_len": PAGED["q_lens"][0],
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
    """The glm16k chunk (c3 shapes and top-k) over an FP8 latent with per-row scales: each
    routing's FP8 entry point (the exact decode into the bf16 workspace, then the attention
    with the row scales) timed as a whole, plus the decode pass alone."""
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
    calls = {
        "decode": [("decode_fp8", lambda: _lib.dsa_decode_latent_fp8(kv8, ws, stream=stream))],
        "grouped": [
            ("build_union", lambda: _lib.dsa_build_group_union(topk, S, 0, G, bufs.union_idx, bufs.union_len,
                                                               bufs.mask, stream=stream)),
            ("grouped_fp8", lambda: _lib.dsa_sparse_prefill_grouped_fp8(q, kv8, ksc, bufs.union_idx, bufs.union_len,
                                                                        bufs.mask, cfg.scale, ws, out_g, lse_g,
                                                                        stream=stream))],
        "per-token": [("pertoken_fp8", lambda: _lib.dsa_sparse_prefill_pertoken_fp8(q, kv8, ksc, topk, 0, cfg.scale,
                                                                                   ws, out_p, lse_p,
                                                                                   stream=stream))],
    }
    samples = {}
    for cl in calls.values():
        smp, _ = time_calls(cl, stream, a.steps, a.warmup)
        samples.update(smp)
    work, nsel = mqa_work(cfg, case.topk, bufs.union_len.cpu().numpy())
    work["decode_fp8"] = ("hbm", S * cfg.d_qk * 3)
    work["grouped_fp8"] = work["grouped_attn"]
    work["pertoken_fp8"] = work["pertoken_attn"]
    routings_out = {}
    for r, cl in calls.items():
        ks = {k: kernel_record(samples[k], *work[k]) for k, _ in cl}
        routings_out[r] = routing_summary(T, ks)
    ms_step = routings_out["grouped"]["ms"]
    d = routings_out["grouped"]["kernels"]["grouped_fp8"]
    line = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8 latent, bf16 compute", "data": "synthetic",
        "config": {"workload": "glm16k_fp8", "routing": "grouped", "T": T, "S": S, "H": H, "k": cfg.k, "G": G,
                   "d_qk": cfg.d_qk, "fp8": "E4M3, per-row float32 scale", "selected_rows": nsel},
        "roofline": {"kernel": "grouped_fp8", "bound": d["bound"], "achieved": round(d["achieved"], 2),
                     "peak": d["peak"], "unit": d["unit"], "frac": round(d["frac"], 4), "traffic": None},
        "cpu_baseline": None,
        "routings": rounded(routings_out),
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
