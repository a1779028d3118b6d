"""Parity at the full workload sizes, in the launch configuration bench.py times.

* union list / length / mask: bit-exact over every group (oracle over all groups);
* grouped and per-token attention: sampled tokens (head and tail of the
  sequence, the partial last group, random tokens) against the fp64 oracle;
* grouped == per-token over every token, checked on the GPU outputs;
* masked MHA: sampled tokens against the dense-mask oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_case
from tests.gpu_helpers import check_attention, check_rows_equal, check_union_rows, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu

MQA = ["c2_dsv32", "c3_glm16k", "c3w_glm16k_uniform", "c5_long", "c7_glm16k_latent512"]


@pytest.fixture(scope="module", params=MQA)
def full(request):
    """Inputs and GPU outputs of one configuration (module-scoped: pytest groups tests by it)."""
    name = request.param
    print(f"[{name}] generating inputs and running both routings", flush=True)
    yield name, _run(name)
    torch.cuda.empty_cache()


def _run(name):
    from mla_prefill_amd import routings
    c = make_case(CONFIGS[name])
    cfg = c.cfg
    q, kv, tk = dev_bf16(c.q), dev_bf16(c.kv), dev_i32(c.topk)
    og, lg, bufs = routings.grouped(q, kv, tk, cfg.q_pos_offset, cfg.scale)
    op, lp = routings.pertoken(q, kv, tk, cfg.q_pos_offset, cfg.scale)
    torch.cuda.synchronize()
    return c, (og, lg), (op, lp), bufs


def sample_tokens(T, G, n_random=48, seed=0):
    rng = np.random.default_rng(seed)
    last_group = ((T - 1) // G) * G
    toks = set(range(0, min(T, 4))) | set(range(max(0, T - 4), T)) | set(range(last_group, T))
    toks |= set(rng.choice(T, size=min(T, n_random), replace=False).tolist())
    return sorted(toks)


def test_union_full(full):
    name, (c, _, _, bufs) = full
    cfg = c.cfg
    print(f"[{name}] union oracle over {cfg.NG} groups", flush=True)
    ui, ul, mk = oracle.group_union_mask(c.topk, cfg.S, cfg.q_pos_offset, cfg.G)
    np.testing.assert_array_equal(bufs.union_len.cpu().numpy(), ul)
    check_union_rows(bufs.union_idx, bufs.mask, ui, ul, mk)


def test_attention_sampled(full):
    name, (c, (og, lg), (op, lp), _) = full
    cfg = c.cfg
    toks = sample_tokens(cfg.T, cfg.G)
    print(f"[{name}] oracle on {len(toks)} sampled tokens", flush=True)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa(c.q, c.kv, c.topk, cfg.S, cfg.q_pos_offset, cfg.scale,
                                                  tokens=toks)
    idx = torch.tensor(toks, device="cuda")
    check_attention(op[idx], lp[idx], ref_out, ref_lse, f"{name} per-token")
    check_attention(og[idx], lg[idx], ref_out, ref_lse, f"{name} grouped")


def test_grouped_equals_pertoken_everywhere(full):
    name, (_, (og, lg), (op, lp), _) = full
    check_rows_equal(og, op, f"{name} grouped vs per-token")
    fin = torch.isfinite(lp)
    assert torch.equal(fin, torch.isfinite(lg))
    assert (lg[fin] - lp[fin]).abs().max().item() <= 2e-3


@pytest.mark.parametrize("name", ["c4_masked_nope", "c6_masked_rope", "c8_masked_dsv32"])
def test_masked_mha_full(name):
    from mla_prefill_amd import routings
    c = make_case(CONFIGS[name])
    cfg = c.cfg
    kp = None if c.k_pe is None else dev_bf16(c.k_pe)
    out, lse, ws = routings.masked_mha(dev_bf16(c.q), dev_bf16(c.k_nope), kp, dev_bf16(c.v),
                                       dev_i32(c.topk), cfg.q_pos_offset, cfg.scale)
    torch.cuda.synchronize()
    toks = sample_tokens(cfg.T, cfg.G, n_random=32, seed=1)
    print(f"[{name}] dense-mask oracle on {len(toks)} sampled tokens", flush=True)
    ref_out, ref_lse = oracle.masked_mha(c.q, c.k_nope, c.k_pe, c.v, c.topk, cfg.S, cfg.q_pos_offset,
                                         cfg.scale, tokens=toks)
    idx = torch.tensor(toks, device="cuda")
    check_attention(out[idx], lse[idx], ref_out, ref_lse, f"{name} masked MHA")
    # bit-packed selection rows of the sampled tokens
    wsn = ws.cpu().numpy().view(np.uint32)
    for t in toks[:8]:
        row = np.zeros(wsn.shape[1], np.uint32)
        for x in oracle.selected_positions(c.topk[t], cfg.S, cfg.q_pos_offset + t):
            row[x // 32] |= np.uint32(1) << np.uint32(x % 32)
        np.testing.assert_array_equal(wsn[t], row)


def test_dense_mha_full():
    """The dense shortcut at its limit, a 2048-token chunk with k = 2048 (16 heads, NoPE
    256): sampled tokens against the oracle, and every output bit-equal to the masked
    kernel's with each token's top-k holding all of its causal keys."""
    from mla_prefill_amd import routings
    from synth.gen import normal_bf16, topk_uniform
    T = S = 2048
    H = 16
    rng = np.random.default_rng(8)
    qn, kn, vn = (normal_bf16(rng, (T, H, 256)) for _ in range(3))
    topk = topk_uniform(rng, T, S, 2048, 2048)
    q, k, v = dev_bf16(qn), dev_bf16(kn), dev_bf16(vn)
    od, ld = routings.dense_mha(q, k, None, v, 0, 1.0 / 16.0)
    om, lm, _ = routings.masked_mha(q, k, None, v, dev_i32(topk), 0, 1.0 / 16.0)
    torch.cuda.synchronize()
    assert torch.equal(od, om) and torch.equal(ld, lm)
    toks = sample_tokens(T, 8, n_random=16, seed=2)
    print(f"[dense 2048] causal oracle on {len(toks)} sampled tokens", flush=True)
    ref_out, ref_lse = oracle.dense_causal_mha(qn, kn, None, vn, S, 0, 1.0 / 16.0, tokens=toks)
    idx = torch.tensor(toks, device="cuda")
    check_attention(od[idx], ld[idx], ref_out, ref_lse, "dense MHA 2048")


def test_fp8_latent_full():
    """The benchmark's FP8 workload: the c3 chunk over an E4M3 latent with per-row scales.
    Sampled tokens of both routings against the oracle, grouped == per-token everywhere."""
    from mla_prefill_amd import routings
    from synth import normal_fp8
    c = make_case(CONFIGS["c3_glm16k"])
    cfg = c.cfg
    codes, kscale = normal_fp8(np.random.default_rng(9), cfg.S, cfg.d_qk, per_row=True)
    q, tk = dev_bf16(c.q), dev_i32(c.topk)
    c8 = torch.from_numpy(codes).cuda()
    s8 = torch.from_numpy(kscale).cuda()
    op, lp = routings.pertoken_fp8(q, c8, s8, tk, 0, cfg.scale)
    og, lg, _ = routings.grouped_fp8(q, c8, s8, tk, 0, cfg.scale)
    torch.cuda.synchronize()
    toks = sample_tokens(cfg.T, cfg.G, n_random=16, seed=4)
    print(f"[fp8] oracle on {len(toks)} sampled tokens", flush=True)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_fp8(c.q, codes, kscale, c.topk, cfg.S, 0, cfg.scale,
                                                      tokens=toks)
    idx = torch.tensor(toks, device="cuda")
    check_attention(op[idx], lp[idx], ref_out, ref_lse, "fp8 per-token")
    check_attention(og[idx], lg[idx], ref_out, ref_lse, "fp8 grouped")
    check_rows_equal(og, op, "fp8 grouped vs per-token")


def test_paged_batch_full():
    """The benchmark's paged batch (8 requests x 2048 query tokens after 14336 positions of
    context, 64-row pages shuffled over a 135168-row cache): union, mask and group table of
    sampled groups bit-exact, both routings on sampled tokens, the index conversion on
    sampled rows."""
    import bench
    from mla_prefill_amd import _lib, routings
    from synth import make_varlen_case
    c = make_varlen_case(**bench.PAGED)
    q, kv, tk = dev_bf16(c.q), dev_bf16(c.kv_cache), dev_i32(c.topk)
    batch = (dev_i32(c.cu_seqlens), dev_i32(c.kv_lens), dev_i32(c.q_pos_start), dev_i32(c.block_table),
             c.page_size)
    og, lg, bufs = routings.grouped_varlen(q, kv, tk, batch, c.scale, max_groups=c.max_groups())
    op, lp, ws = routings.pertoken_varlen(q, kv, tk, batch, c.scale)
    torch.cuda.synchronize()
    args = (c.cu_seqlens, c.kv_lens, c.q_pos_start, c.block_table, c.page_size)
    groups = oracle.varlen_groups(c.cu_seqlens, c.G)
    rng = np.random.default_rng(3)
    pick = sorted(set([0, 255, 256, len(groups) - 1]) | set(rng.choice(len(groups), 28, replace=False).tolist()))
    print(f"[paged] union oracle on {len(pick)} groups, attention on their tokens", flush=True)
    info, ui, ul, mk = (x.cpu().numpy() for x in (bufs.group_info, bufs.union_idx, bufs.union_len, bufs.mask))
    toks = []
    for g in pick:
        t0, n = groups[g]
        np.testing.assert_array_equal(info[g], (t0, n))
        r = int(np.searchsorted(c.cu_seqlens, t0, side="right") - 1)
        sub = (np.array([0, n]), c.kv_lens[r:r + 1], c.q_pos_start[r:r + 1] + (t0 - c.cu_seqlens[r]),
               c.block_table[r:r + 1], c.page_size)
        _, ui1, ul1, mk1 = oracle.group_union_mask_varlen(c.topk[t0:t0 + n], *sub, c.num_slots, c.G, 1,
                                                          pad=ui.shape[1])
        assert ul[g] == ul1[0]
        check_union_rows(ui[g:g + 1], mk[g:g + 1], ui1, ul1, mk1, f"paged group {g}")
        toks.extend(range(t0, t0 + n))
    # index conversion of request 0's first 64 tokens
    ref_g = oracle.convert_req_index_to_global(c.topk[:64], np.array([0, 64]), c.kv_lens[:1],
                                               c.q_pos_start[:1], c.block_table[:1], c.page_size, c.num_slots)
    np.testing.assert_array_equal(ws[:64].cpu().numpy(), ref_g)
    ref_out, ref_lse = oracle.pertoken_sparse_mqa_varlen(c.q, c.kv_cache, c.topk, *args, c.scale, tokens=toks)
    idx = torch.tensor(toks, device="cuda")
    check_attention(og[idx], lg[idx], ref_out, ref_lse, "paged grouped")
    check_attention(op[idx], lp[idx], ref_out, ref_lse, "paged per-token")
