"""Seeded generators for the DSA sparse-prefill workloads.

Everything here is input drawing: bf16 values as uint16 bit patterns and
int32 top-k index buffers padded with -1.  The arithmetic of the attention
method lives elsewhere (the CPU oracle and the HIP kernels), and this module
shares none of it.

Recipe (same for every configuration):

* numpy PCG64, ``SeedSequence(seed).spawn(3)`` gives three independent
  streams: (queries, keys/values, top-k indices).
* Values are float32 N(0, 1) draws rounded to bf16 with round-to-nearest-even.
* Top-k rows hold a random permutation of the token's selected positions,
  then -1 up to the buffer width.  Query token t sits at absolute position
  p(t) = q_pos_offset + t and selects only positions <= p(t).

Top-k structure stands in for the real indexer output on real prompts that
the pages measure on ("the union of 8 adjacent tokens' top-2048 is ~2.4k keys",
Grouped sparse prefill page, commit message and "Why" section):

* ``topk_locality``: a group of G consecutive tokens shares a base set drawn
  uniformly from the causal range of the group's first token; every token then
  swaps 2.5 % of its entries for positions of its own causal range outside the
  set.  With G = 8 and k = 2048 the full-group union is ~2.45k.
* ``topk_uniform``: every token draws its own set uniformly from its causal
  range (the worst case for the union).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_CHUNK = 1 << 24  # values drawn per standard_normal call (fixed for determinism)


# ---------------------------------------------------------------------------
# bf16 bit patterns
# ---------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) float32 draws rounded to bf16, returned as uint16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = bf16_bits_from_f32(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


def normal_fp8(rng: np.random.Generator, rows: int, d: int, per_row: bool = True):
    """An FP8 latent: N(0, 1) float32 draws stored as OCP E4M3 codes (uint8 [rows, d]) with
    float32 scales (per row: the row's largest magnitude / 448, else one for the whole
    tensor), encoded by torch's float8_e4m3fn conversion (nearest even).  Returns
    (codes, scales [rows] or [1])."""
    import torch
    v = rng.standard_normal((rows, d), dtype=np.float32)
    amax = np.abs(v).max(axis=1) if per_row else np.array([np.abs(v).max()], np.float32)
    scale = (np.maximum(amax, 1e-30) / np.float32(448.0)).astype(np.float32)
    x = v / (scale[:, None] if per_row else scale[0])
    codes = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


# ---------------------------------------------------------------------------
# top-k index buffers
# ---------------------------------------------------------------------------

def topk_uniform(rng: np.random.Generator, T: int, S: int, k: int, cols: int,
                 q_pos_offset: int = 0) -> np.ndarray:
    """Each token draws min(k, p+1) distinct positions uniformly from [0, p]."""
    if cols < k:
        raise ValueError("cols must be >= k")
    out = np.full((T, cols), -1, dtype=np.int32)
    for t in range(T):
        p = q_pos_offset + t
        if p >= S:
            raise ValueError("query position beyond the KV length")
        n = min(k, p + 1)
        out[t, :n] = rng.choice(p + 1, size=n, replace=False)
    return out


def _non_members(s: np.ndarray, p: int) -> np.ndarray:
    member = np.zeros(p + 1, dtype=bool)
    member[s] = True
    return np.flatnonzero(~member)


def topk_locality(rng: np.random.Generator, T: int, S: int, k: int, cols: int, G: int,
                  q_pos_offset: int = 0, resample_frac: float = 0.025) -> np.ndarray:
    """Group-local top-k sets.

    Per group of G consecutive tokens (first token t0, p0 = P0 + t0):
      1. base set B: min(k, p0 + 1) positions uniform without replacement from [0, p0];
      2. token t (n = min(k, p(t) + 1)) starts from B, topped up uniformly from
         [0, p(t)] minus B when |B| < n;
      3. when p(t) + 1 > n, r = min(floor(resample_frac * n), p(t) + 1 - n) uniformly
         chosen members are replaced by as many uniformly chosen non-members of
         [0, p(t)] (the cap only matters just past the top-k budget, where fewer than
         floor(resample_frac * n) non-members exist);
      4. the row is a random permutation of the set, then -1 up to ``cols``.
    """
    if cols < k:
        raise ValueError("cols must be >= k")
    out = np.full((T, cols), -1, dtype=np.int32)
    for t0 in range(0, T, G):
        p0 = q_pos_offset + t0
        base = rng.choice(p0 + 1, size=min(k, p0 + 1), replace=False).astype(np.int64)
        for t in range(t0, min(T, t0 + G)):
            p = q_pos_offset + t
            if p >= S:
                raise ValueError("query position beyond the KV length")
            n = min(k, p + 1)
            s = base
            if s.size < n:
                extra = rng.choice(_non_members(s, p), size=n - s.size, replace=False)
                s = np.concatenate([s, extra])
            if p + 1 > n:
                r = min(int(math.floor(resample_frac * n)), p + 1 - n)
                if r > 0:
                    drop = rng.choice(n, size=r, replace=False)
                    add = rng.choice(_non_members(s, p), size=r, replace=False)
                    s = s.copy()
                    s[drop] = add
            out[t, :n] = s[rng.permutation(n)]
    return out


def shuffle_rows(topk: np.ndarray, seed: int) -> np.ndarray:
    """Permute every row's columns (moves the -1 padding to random places)."""
    rng = np.random.default_rng(seed)
    out = topk.copy()
    for t in range(out.shape[0]):
        out[t] = out[t, rng.permutation(out.shape[1])]
    return out


def widen(topk: np.ndarray, cols: int) -> np.ndarray:
    """Append -1 columns up to ``cols``."""
    out = np.full((topk.shape[0], cols), -1, dtype=np.int32)
    out[:, :topk.shape[1]] = topk
    return out


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    T: int
    S: int
    H: int
    k: int
    cols: int
    G: int
    scale: float
    seed: int
    q_pos_offset: int = 0
    topk_mode: str = "locality"          # "locality" | "uniform"
    kind: str = "mqa"                    # "mqa" (576-wide latent) | "mha" (per-head K/V)
    d_qk: int = 576
    d_v: int = 512
    dn: int = 0                          # masked MHA: nope width of q/k
    dr: int = 0                          # masked MHA: rope width (shared k_pe)
    dv: int = 0                          # masked MHA: value width
    note: str = ""

    @property
    def NG(self) -> int:
        return -(-self.T // self.G)

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # Tiny sparse MQA prefill; uniform top-32 from the causal range.
    "c1_tiny": Config("c1_tiny", T=64, S=64, H=16, k=32, cols=32, G=8,
                      scale=1.0 / math.sqrt(192.0), seed=0, topk_mode="uniform"),
    # DeepSeek-V3.2-style layer: 128 heads, group of 1 token.
    "c2_dsv32": Config("c2_dsv32", T=4096, S=4096, H=128, k=2048, cols=2048, G=1,
                       scale=1.0 / math.sqrt(192.0), seed=1),
    # GLM-style per-GPU share: 16 heads, 16k chunk, groups of 8 tokens.
    "c3_glm16k": Config("c3_glm16k", T=16384, S=16384, H=16, k=2048, cols=2048, G=8,
                        scale=1.0 / 16.0, seed=2),
    # Same shapes, uniform top-k (worst case for the union).
    "c3w_glm16k_uniform": Config("c3w_glm16k_uniform", T=16384, S=16384, H=16, k=2048,
                                 cols=2048, G=8, scale=1.0 / 16.0, seed=2,
                                 topk_mode="uniform"),
    # Masked dense MHA over the NoPE layout (qk 256, rope 0, v 256).
    "c4_masked_nope": Config("c4_masked_nope", T=16384, S=16384, H=16, k=2048, cols=2048,
                             G=8, scale=1.0 / 16.0, seed=3, kind="mha", d_qk=256, d_v=256,
                             dn=256, dr=0, dv=256),
    # Masked dense MHA with a rope part (qk 256 = nope 192 + shared rope 64, v 256), the
    # other layout the qk 256 / v 256 kernel serves; same shapes and top-k recipe as c4.
    "c6_masked_rope": Config("c6_masked_rope", T=16384, S=16384, H=16, k=2048, cols=2048,
                             G=8, scale=1.0 / 16.0, seed=5, kind="mha", d_qk=256, d_v=256,
                             dn=192, dr=64, dv=256),
    # The 512-wide latent (no rope part; K = V = the whole row), the MQA form of the NoPE
    # (256, 0, 256) model; otherwise the shapes and top-k recipe of c3.
    "c7_glm16k_latent512": Config("c7_glm16k_latent512", T=16384, S=16384, H=16, k=2048,
                                  cols=2048, G=8, scale=1.0 / 16.0, seed=7, d_qk=512),
    # Masked dense MHA in the DeepSeek-V3.2 geometry (qk 192 = nope 128 + shared rope 64,
    # v 128) at 128 heads, over the chunk and top-k recipe of c2.
    "c8_masked_dsv32": Config("c8_masked_dsv32", T=4096, S=4096, H=128, k=2048, cols=2048, G=1,
                              scale=1.0 / math.sqrt(192.0), seed=8, kind="mha", d_qk=192, d_v=128,
                              dn=128, dr=64, dv=128),
    # Long prompt: the last 21504 of 32768 positions are queries; 2176-wide top-k buffer.
    "c5_long": Config("c5_long", T=21504, S=32768, H=16, k=2048, cols=2176, G=8,
                      scale=1.0 / 16.0, seed=4, q_pos_offset=11264),
}


@dataclass
class Case:
    cfg: Config
    topk: np.ndarray                       # int32 [T, cols]
    q: Optional[np.ndarray] = None         # uint16 bf16 bits
    kv: Optional[np.ndarray] = None        # mqa: [S, 576]
    k_nope: Optional[np.ndarray] = None    # mha: [S, H, dn]
    k_pe: Optional[np.ndarray] = None      # mha: [S, dr] or None
    v: Optional[np.ndarray] = None         # mha: [S, H, dv]
    extra: dict = field(default_factory=dict)


def make_topk(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.topk_mode == "uniform":
        return topk_uniform(rng, cfg.T, cfg.S, cfg.k, cfg.cols, cfg.q_pos_offset)
    if cfg.topk_mode == "locality":
        return topk_locality(rng, cfg.T, cfg.S, cfg.k, cfg.cols, cfg.G, cfg.q_pos_offset)
    raise ValueError(cfg.topk_mode)


def make_case(cfg: Config, values: bool = True) -> Case:
    """Draw every input of ``cfg`` from its seed (see the module docstring)."""
    if cfg.q_pos_offset + cfg.T > cfg.S:
        raise ValueError("q_pos_offset + T must not exceed S")
    ss = np.random.SeedSequence(cfg.seed).spawn(3)
    rq, rkv, rtk = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    case = Case(cfg=cfg, topk=make_topk(cfg, rtk))
    if not values:
        return case
    if cfg.kind == "mqa":
        case.q = normal_bf16(rq, (cfg.T, cfg.H, cfg.d_qk))
        case.kv = normal_bf16(rkv, (cfg.S, cfg.d_qk))
    elif cfg.kind == "mha":
        case.q = normal_bf16(rq, (cfg.T, cfg.H, cfg.dn + cfg.dr))
        case.k_nope = normal_bf16(rkv, (cfg.S, cfg.H, cfg.dn))
        case.k_pe = normal_bf16(rkv, (cfg.S, cfg.dr)) if cfg.dr > 0 else None
        case.v = normal_bf16(rkv, (cfg.S, cfg.H, cfg.dv))
    else:
        raise ValueError(cfg.kind)
    return case


# ---------------------------------------------------------------------------
# batches of requests over a paged KV cache
# ---------------------------------------------------------------------------

@dataclass
class VarlenCase:
    q: np.ndarray             # uint16 bf16 bits [T, H, d_qk], requests' tokens concatenated
    kv_cache: np.ndarray      # uint16 bf16 bits [num_slots, d_qk] (pages of page_size rows)
    topk: np.ndarray          # int32 [T, cols], request-local positions, -1 padded
    cu_seqlens: np.ndarray    # int32 [R + 1]
    kv_lens: np.ndarray       # int32 [R]
    q_pos_start: np.ndarray   # int32 [R]: position of each request's first query token
    block_table: np.ndarray   # int32 [R, max_pages]: physical page of each request page (-1 unused)
    page_size: int
    scale: float
    G: int

    @property
    def num_slots(self) -> int:
        return self.kv_cache.shape[0]

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    def max_groups(self) -> int:
        return int(sum(-(-int(n) // self.G) for n in np.diff(self.cu_seqlens)))


def make_varlen_case(seed: int, q_lens, ctx_lens, H: int = 16, k: int = 2048, cols: int = 0,
                     page_size: int = 64, G: int = 8, mode: str = "locality", spare_pages: int = 3,
                     d_qk: int = 576, scale: float = 1.0 / 16.0, values: bool = True) -> VarlenCase:
    """A seeded batch: request r has q_lens[r] query tokens after ctx_lens[r] positions of
    context (kv_len = ctx + q_len, first query position = ctx).  The cache holds every
    request's pages plus ``spare_pages`` unused ones, in a random physical order; each
    request's top-k rows come from the single-sequence generators over its own positions."""
    q_lens = [int(n) for n in q_lens]
    ctx_lens = [int(c) for c in ctx_lens]
    R = len(q_lens)
    cols = cols or k
    ss = np.random.SeedSequence(seed).spawn(4)
    rq, rkv, rtk, rpg = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    cu = np.zeros(R + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    kv_lens = np.asarray([c + n for c, n in zip(ctx_lens, q_lens)], dtype=np.int32)
    q_pos_start = np.asarray(ctx_lens, dtype=np.int32)
    pages = [-(-int(L) // page_size) for L in kv_lens]
    total_pages = sum(pages) + spare_pages
    perm = rpg.permutation(total_pages).astype(np.int32)
    block_table = np.full((R, max(1, max(pages) if pages else 1)), -1, dtype=np.int32)
    at = 0
    for r in range(R):
        block_table[r, :pages[r]] = perm[at:at + pages[r]]
        at += pages[r]
    parts = []
    for r in range(R):
        n, L, c = q_lens[r], int(kv_lens[r]), ctx_lens[r]
        if mode == "uniform":
            parts.append(topk_uniform(rtk, n, L, k, cols, c))
        else:
            parts.append(topk_locality(rtk, n, L, k, cols, G, c))
    topk = np.concatenate(parts, axis=0) if parts else np.zeros((0, cols), np.int32)
    T = int(cu[-1])
    case = VarlenCase(q=None, kv_cache=None, topk=topk, cu_seqlens=cu, kv_lens=kv_lens,
                      q_pos_start=q_pos_start, block_table=block_table, page_size=page_size,
                      scale=scale, G=G)
    if values:
        case.q = normal_bf16(rq, (T, H, d_qk))
        case.kv_cache = normal_bf16(rkv, (total_pages * page_size, d_qk))
    else:
        case.kv_cache = np.zeros((total_pages * page_size, 0), np.uint16)
    return case
