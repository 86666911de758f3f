"""Parity of the HIP path (through the C ABI) with the oracle, stage by stage
and end to end. Every stage is fed the same inputs on both sides; integer
tables, permutations and FP8 bytes must match exactly, bf16 results within
atol = rtol = 1e-2, routing weights within 2e-6 relative.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from oracle import numerics as nm
from gpu_util import (BF16_ATOL, BF16_RTOL, assert_bf16_close, bf16_ulp, bits, dev, host, inputs, oracle_tokens,
                      say)

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mixture_experts_routed_moe_amd")

MID = moe_synth.MoEConfig(80, "mid", T=300, H=256, F=384, E=6, top_k=2, padding_m=128, block_m=128)
MID64 = moe_synth.MoEConfig(81, "mid64", T=300, H=256, F=384, E=6, top_k=2, padding_m=128, block_m=64)


def _t(a, d, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(d)


def _bf16_dev(bits_np, d):
    return torch.from_numpy(np.ascontiguousarray(bits_np).view(np.int16)).view(torch.bfloat16).to(d)


# ---------------------------------------------------------------- inputs --

def test_generator_same_bits_on_gpu():
    d = dev()
    key = moe_synth.tensor_key(3, 4)
    a = moe_synth.normal_bf16(key, (5000,), 0.02, "cpu", start=123456)
    b = moe_synth.normal_bf16(key, (5000,), 0.02, d, start=123456)
    assert torch.equal(a, b.cpu())
    cfg = moe_synth.CONFIGS["qwen3_decode"]
    assert torch.equal(moe_synth.router_logits(cfg, "cpu", rows=slice(7, 11)),
                       moe_synth.router_logits(cfg, d, rows=slice(7, 11)).cpu())


# --------------------------------------------------------------- routing --

@pytest.mark.parametrize("name", ["tiny", "qwen3_decode", "qwen3_prefill", "dsv3_prefill", "kimi_k2_t4096"])
def test_route(name):
    d = dev()
    cfg = moe_synth.CONFIGS[name]
    say("route", name)
    logits = moe_synth.router_logits(cfg, d)
    bias = moe_synth.expert_bias(cfg, d)
    ids, w = mx.moe_topk_softmax(logits, cfg.top_k, expert_bias=bias, scoring=cfg.scoring,
                                 renormalize=cfg.renormalize)
    rid, rw = oracle.route(host(logits), cfg.top_k, None if bias is None else host(bias), cfg.scoring,
                           cfg.renormalize)
    assert np.array_equal(host(ids), rid)
    np.testing.assert_allclose(host(w), rw, rtol=2e-6, atol=1e-7)


def test_route_ties_and_small_shapes():
    d = dev()
    rng = np.random.default_rng(3)
    for T, E, k in [(37, 8, 2), (5, 3, 3), (64, 1024, 16), (9, 65, 7), (1, 1, 1)]:
        logits = rng.integers(-3, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)
        ids, w = mx.moe_topk_softmax(_t(logits, d), k)
        rid, rw = oracle.route(logits, k)
        assert np.array_equal(host(ids), rid), (T, E, k)
        np.testing.assert_allclose(host(w), rw, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_route_signed_zero_ties_and_infinities(scoring):
    """The argmax rounds compare order-preserving codes of the logits: -0 and
    +0 tie (the lower id first, as the oracle's stable sort), -inf entries
    rank last, large magnitudes keep their order."""
    d = dev()
    rng = np.random.default_rng(4)
    T, E, k = 64, 200, 8
    vals = np.array([0.0, -0.0, -np.inf, 3.0e38, -3.0e38, 1.0e-38, -1.0e-38, 0.5, -0.5], np.float32)
    logits = vals[rng.integers(0, vals.size, size=(T, E))]
    logits[:, 0] = np.float32(-0.0)          # every row holds signed zeros and at least one finite logit
    logits[0] = np.float32(-0.0)             # a row of -0 only
    logits[1, ::2] = np.float32(0.0)         # alternating +0 / -0
    logits[1, 1::2] = np.float32(-0.0)
    logits[2] = -np.inf
    logits[2, 150:] = np.float32(-0.0)       # -inf everywhere but 50 zeros
    ids, w = mx.moe_topk_softmax(_t(logits, d), k, scoring=scoring)
    rid, rw = oracle.route(logits, k, None, scoring)
    assert np.array_equal(host(ids), rid)
    np.testing.assert_allclose(host(w), rw, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renormalize", [True, False])
def test_route_scoring_bias_renormalize(scoring, renormalize):
    d = dev()
    rng = np.random.default_rng(11)
    for T, E, k in [(300, 384, 8), (77, 64, 6), (5, 1000, 16)]:
        logits = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
        for bias in (None, (rng.standard_normal(E) * 2).astype(np.float32)):
            ids, w = mx.moe_topk_softmax(_t(logits, d), k, expert_bias=None if bias is None else _t(bias, d),
                                         scoring=scoring, renormalize=renormalize)
            rid, rw = oracle.route(logits, k, bias, scoring, renormalize)
            assert np.array_equal(host(ids), rid), (T, E, k, bias is None)
            np.testing.assert_allclose(host(w), rw, rtol=2e-6, atol=1e-7)


# ------------------------------------------------------------ dispatch --

def _align_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dispatch_worked_example.json")))
    p = g["params"]
    yield "worked", np.array(g["topk_ids"], np.int32), p["experts"], p["padding_m"], p["block_token"]
    rng = np.random.default_rng(0)
    yield "empty", np.zeros((0, 2), np.int32), 4, 64, 64
    yield "one_expert", np.full((300, 1), 5, np.int32), 8, 128, 128
    yield "exact_multiples", np.repeat(np.arange(4, dtype=np.int32), 64).reshape(-1, 2), 4, 64, 64
    yield "pad128_block64", np.stack([rng.permutation(16)[:4] for _ in range(777)]).astype(np.int32), 16, 128, 64
    yield "E1", np.zeros((50, 1), np.int32), 1, 16, 16
    yield "E1000", np.stack([rng.permutation(1000)[:8] for _ in range(2100)]).astype(np.int32), 1000, 32, 32
    # around the one-launch form's limit of two 1024-pair chunks
    yield "two_chunks", np.stack([rng.permutation(64)[:2] for _ in range(750)]).astype(np.int32), 64, 128, 128
    yield "2048_pairs", np.stack([rng.permutation(48)[:2] for _ in range(1024)]).astype(np.int32), 48, 128, 128
    yield "2049_pairs", rng.integers(0, 48, (2049, 1)).astype(np.int32), 48, 128, 64
    yield "E1000_two_chunks", np.stack([rng.permutation(1000)[:2] for _ in range(1000)]).astype(np.int32), 1000, 128, 128
    yield "eight_chunks", np.stack([rng.permutation(32)[:8] for _ in range(1024)]).astype(np.int32), 32, 128, 128
    for name in ("tiny", "qwen3_decode", "qwen3_prefill", "dsv3_prefill", "kimi_k2_t4096"):
        cfg = moe_synth.CONFIGS[name]
        bias = moe_synth.expert_bias(cfg)
        ids, _ = oracle.route(moe_synth.router_logits(cfg).numpy(), cfg.top_k, None if bias is None else bias.numpy(),
                              cfg.scoring, cfg.renormalize)
        yield name, ids, cfg.E, cfg.padding_m, cfg.block_m


def test_align_tables_bit_exact(golden_dir):
    d = dev()
    for name, ids, E, pm, bm in _align_cases(golden_dir):
        say("align", name, ids.shape, E, pm, bm)
        tb = mx.moe_align(_t(ids, d), E, pm, bm)
        ref = oracle.dispatch_tables(ids, E, pm, bm)
        for key in ("group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                    "sorted_pair", "pair_to_row"):
            assert np.array_equal(host(tb[key]), ref[key]), (name, key)
        assert tb["group_idx_for_bx"].numel() == ref["m_blocks"]


def test_align_deterministic():
    d = dev()
    cfg = moe_synth.CONFIGS["dsv3_prefill"]
    ids, _ = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), cfg.top_k,
                                 expert_bias=moe_synth.expert_bias(cfg, d))
    a = mx.moe_align(ids, cfg.E, cfg.padding_m, cfg.block_m)
    b = mx.moe_align(ids, cfg.E, cfg.padding_m, cfg.block_m)
    for key in ("sorted_pair", "pair_to_row", "group_idx_for_bx"):
        assert torch.equal(a[key], b[key])


@pytest.mark.parametrize("T,k,E,skew", [(262145, 8, 256, True), (300001, 7, 1000, False), (2100000, 1, 3, False)])
def test_align_large_bit_exact(T, k, E, skew):
    """Past 2^21 pairs (2049-2051 chunks of 1024 pairs, the last one ragged),
    against the oracle's tables: the scan over chunks runs in ranges across
    16 waves, whose boundaries fall inside the chunk sequence."""
    d = dev()
    say("align large", T, k, E, skew)
    rng = np.random.default_rng(T)
    if skew:
        # Zipf-like expert popularity: some experts empty, a few very large
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p[rng.choice(E, E // 8, replace=False)] = 0.0
        p /= p.sum()
        ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(64)]).astype(np.int32)
        ids = ids[rng.integers(0, 64, T)]
    else:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32) if E <= 8 else \
            np.stack([rng.permutation(E)[:k] for _ in range(97)]).astype(np.int32)[rng.integers(0, 97, T)]
    tb = mx.moe_align(_t(ids, d), E, 128, 128)
    ref = oracle.dispatch_tables(ids, E, 128, 128)
    for key in ("group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                "sorted_pair", "pair_to_row"):
        assert np.array_equal(host(tb[key]), ref[key]), key


# ------------------------------------------------------------- permute --

@pytest.mark.parametrize("name", ["tiny", "qwen3_prefill", "dsv3_prefill"])
def test_permute(name):
    d = dev()
    cfg = moe_synth.CONFIGS[name]
    hid = moe_synth.hidden(cfg, d)
    ids, _ = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), cfg.top_k,
                                 expert_bias=moe_synth.expert_bias(cfg, d))
    tb = mx.moe_align(ids, cfg.E, cfg.padding_m, cfg.block_m)
    ref = oracle.permute(bits(hid), host(tb["sorted_pair"]), cfg.top_k)
    # gather by sorted_pair, scatter by pair_to_row, and both given (scatter)
    for sp, p2r in ((tb["sorted_pair"], None), (None, tb["pair_to_row"]), (tb["sorted_pair"], tb["pair_to_row"])):
        xp = mx.moe_permute(hid, sp, cfg.top_k, pair_to_row=p2r)
        assert np.array_equal(bits(xp), ref), (sp is None, p2r is None)


@pytest.mark.parametrize("T,k,H,E", [(7, 3, 200, 5), (37, 16, 64, 40), (5, 2, 16392, 4), (300, 1, 2056, 3)])
def test_permute_ragged_shapes(T, k, H, E):
    """Row counts that are not multiples of the rows per workgroup, rows that
    are not multiples of the 256-chunk pass, rows wider than one pass."""
    d = dev()
    rng = np.random.default_rng(T * 1000 + H)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tb = mx.moe_align(_t(ids, d), E, 16, 16)
    hid = moe_synth.normal_bf16(moe_synth.tensor_key(74, H), (T, H), 1.0, d)
    ref = oracle.permute(bits(hid), host(tb["sorted_pair"]), k)
    for sp, p2r in ((tb["sorted_pair"], None), (None, tb["pair_to_row"])):
        assert np.array_equal(bits(mx.moe_permute(hid, sp, k, pair_to_row=p2r)), ref)


# ---------------------------------------------------------------- GEMMs --

def _gemm_setup(cfg, d):
    hid = moe_synth.hidden(cfg, d)
    ids, w = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), cfg.top_k)
    tb = mx.moe_align(ids, cfg.E, cfg.padding_m, cfg.block_m)
    xp = mx.moe_permute(hid, tb["sorted_pair"], cfg.top_k)
    return xp, tb, ids, w


@pytest.mark.parametrize("cfg", [moe_synth.CONFIGS["tiny"], MID, MID64], ids=["tiny", "mid", "mid64"])
def test_grouped_gemm_gate_up_and_down(cfg):
    d = dev()
    say("gemm", cfg.name)
    xp, tb, _, _ = _gemm_setup(cfg, d)
    wgu = moe_synth.w_gate_up(cfg, d)
    wd = moe_synth.w_down(cfg, d)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    assert (gs % cfg.block_m != 0).any()        # ragged tails exercised
    gu = mx.grouped_gemm_gate_up(xp, wgu, tb, cfg.padding_m, cfg.block_m, fuse_swiglu=False)
    ref_gu = oracle.grouped_gemm(bits(xp), bits(wgu), gs, go)
    err = assert_bf16_close(bits(gu), ref_gu, "gate_up")
    say("  gate_up max abs err", err)
    # fused epilogue == unfused GEMM + SwiGLU, byte for byte, and == the oracle's SwiGLU of it
    h = mx.grouped_gemm_gate_up(xp, wgu, tb, cfg.padding_m, cfg.block_m, fuse_swiglu=True)
    assert torch.equal(h, mx.swiglu(gu))
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), cfg.F))
    y = mx.grouped_gemm_down(h, wd, tb, cfg.padding_m, cfg.block_m)
    ref_y = oracle.grouped_gemm(bits(h), bits(wd), gs, go)
    err = assert_bf16_close(bits(y), ref_y, "down")
    say("  down max abs err", err)


# the gathering gate_up on each kernel path: 64-row blocks (register-staged),
# few rows per expert (128-row pipeline), >= 128 rows per expert (256-row
# kernel), one token's top-k over 160 experts (few-row kernel)
WIDE = moe_synth.MoEConfig(82, "wide", T=2048, H=256, F=384, E=8, top_k=2, padding_m=128, block_m=128)
ONE_TOKEN = moe_synth.MoEConfig(83, "one_token", T=1, H=256, F=384, E=160, top_k=8, padding_m=128, block_m=128)


@pytest.mark.parametrize("cfg", [MID64, MID, WIDE, ONE_TOKEN], ids=["mid64", "mid", "wide", "one_token"])
def test_gate_up_gather_equals_permute_then_gemm(cfg):
    """The permute folded into gate_up's A loads gives the same bytes as
    moe_permute followed by grouped_gemm_gate_up (whose oracle parity the
    tests above establish), fused and unfused; plus the oracle directly on the
    unfused product."""
    d = dev()
    say("gather gemm", cfg.name)
    hid = moe_synth.hidden(cfg, d)
    xp, tb, _, _ = _gemm_setup(cfg, d)
    wgu = moe_synth.w_gate_up(cfg, d)
    for fuse in (True, False):
        ref = mx.grouped_gemm_gate_up(xp, wgu, tb, cfg.padding_m, cfg.block_m, fuse_swiglu=fuse)
        got = mx.grouped_gemm_gate_up_gather(hid, wgu, tb, cfg.top_k, cfg.padding_m, cfg.block_m, fuse_swiglu=fuse)
        assert torch.equal(got, ref), f"fuse={fuse}"
    # the oracle side from the oracle alone: routing, tables, permute, product
    ref_ids, _ = oracle.route(host(moe_synth.router_logits(cfg, d)), cfg.top_k)
    tab = oracle.dispatch_tables(ref_ids, cfg.E, cfg.padding_m, cfg.block_m)
    for key in ("group_sizes", "group_offsets", "sorted_pair"):
        assert np.array_equal(host(tb[key]), tab[key]), key
    ref_xp = oracle.permute(bits(hid), tab["sorted_pair"], cfg.top_k)
    ref_gu = oracle.grouped_gemm(ref_xp, bits(wgu), tab["group_sizes"], tab["group_offsets"])
    assert_bf16_close(bits(got), ref_gu, "gather gate_up")



def test_wide_fused_swiglu_gates_outside_table():
    """The 256-row kernel's fused SwiGLU takes each SiLU from a table of the
    bf16 gates with |g| in [2^-25, 128), the closed forms g/2 and g beyond it,
    and the direct evaluation for a wave holding a gate at or below -128.
    Gates built to land in each range (a constant-1 input column times a
    +-1000 weight, or weights scaled by 1e-9): the fused bytes equal the
    oracle's SwiGLU of the unfused product, and the swiglu kernel's."""
    d = dev()
    cfg = WIDE
    F = cfg.F
    xp, tb, _, _ = _gemm_setup(cfg, d)
    xp = xp.clone()
    xp[:, 0] = 1.0
    w = moe_synth.w_gate_up(cfg, d).clone()
    w[1, 0:32, 0] = 1000.0         # expert 1, gate columns 0-31: about +1000 (closed form g, table path)
    w[2, 64:96, 0] = -1000.0       # expert 2, gate columns 64-95: about -1000 (direct evaluation)
    w[3, 128:160, :] *= 1e-9       # expert 3, gate columns 128-159: below 2^-25 (closed form g/2)
    h = mx.grouped_gemm_gate_up(xp, w, tb, cfg.padding_m, cfg.block_m, fuse_swiglu=True)
    gu = mx.grouped_gemm_gate_up(xp, w, tb, cfg.padding_m, cfg.block_m, fuse_swiglu=False)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    assert gs[1] > 128 and gs[2] > 128 and gs[3] > 128   # the 256-row kernel's tiles
    g = gu[:, :F].float().cpu().numpy()
    rows = lambda e: slice(int(go[e]), int(go[e] + gs[e]))
    assert (g[rows(1), 0:32] >= 128).all()
    assert (g[rows(2), 64:96] <= -128).all()
    tiny = np.abs(g[rows(3), 128:160])
    assert (tiny < 2.0 ** -25).all() and (tiny > 0).any()
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
    assert torch.equal(h, mx.swiglu(gu))

def test_gate_up_gather_past_4gib():
    """Hidden states past 2^32 bytes (T = 300000, H = 7168: 4.3 GB): the
    256-row kernel addresses gathered rows with 32-bit offsets from the
    first hidden row, so this launch must take the 128-row kernel; the
    permuted copy (8.6 GB of x_perm reads and writes) goes through the
    256-row kernel with per-tile offsets. Sampled rows of both against the
    oracle, including the last rows of the array."""
    d = dev()
    T, H, F, E, k = 300_000, 7168, 128, 4, 1
    assert T * H * 2 >= 1 << 32
    say("gather past 4 GiB", T, H)
    key = moe_synth.tensor_key(88)
    hid = moe_synth.normal_bf16(key, (T, H), 1.0, d)
    ids_np = np.random.default_rng(88).integers(0, E, size=(T, k)).astype(np.int32)
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, H), H ** -0.5, d)
    h_g = mx.grouped_gemm_gate_up_gather(hid, wgu, tb, k, 128, 128)
    xp = mx.moe_permute(hid, None, k, pair_to_row=tb["pair_to_row"])
    h_p = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128)
    del xp
    torch.cuda.synchronize()
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    sp = host(tb["sorted_pair"])
    rows = np.unique(np.concatenate([[0, T - 1], go[1:] - 1, go, np.random.default_rng(1).choice(T, 24)]))
    rows = rows[(rows >= 0) & (rows < T)]
    expert = np.searchsorted(np.concatenate([go, [T]]), rows, side="right") - 1
    for e in range(E):
        sel = rows[expert == e]
        if sel.size == 0:
            continue
        a = bits(hid[torch.as_tensor(sp[sel] // k, device=d)])
        ref = oracle.swiglu(oracle.grouped_gemm(a, bits(wgu[e:e + 1]), np.array([sel.size], np.int32),
                                                np.array([0], np.int32)), F)
        got_g = bits(h_g[torch.as_tensor(sel, device=d)])
        got_p = bits(h_p[torch.as_tensor(sel, device=d)])
        assert_bf16_close(got_g, ref, f"gather, expert {e}")
        assert_bf16_close(got_p, ref, f"permuted copy, expert {e}")


@pytest.mark.parametrize("numel,bm", [(1, 64), (200, 128), (333, 64), (4096, 128)])
def test_dense_group_gemm(numel, bm):
    d = dev()
    H, F = 256, 192
    key = moe_synth.tensor_key(70, numel)
    x = moe_synth.normal_bf16(key, (numel, H), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (2 * F, H), H ** -0.5, d)
    wd = moe_synth.normal_bf16(key + 2, (H, F), F ** -0.5, d)
    gu = mx.grouped_gemm_gate_up(x, wgu, None, bm, bm, fuse_swiglu=False)
    one, zero = np.array([numel], np.int32), np.array([0], np.int32)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu)[None], one, zero), "dense gate_up")
    h = mx.grouped_gemm_gate_up(x, wgu, None, bm, bm, fuse_swiglu=True)
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
    y = mx.grouped_gemm_down(h, wd, None, bm, bm)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd)[None], one, zero), "dense down")


# Expert sizes around the 128-row block and the 256-row pair of blocks: an
# empty expert, single rows, partial and exact blocks, odd and even block
# counts (the last block of an odd count is computed on its own).
EDGE_SIZES = [0, 1, 127, 128, 129, 255, 256, 257, 383, 384, 385, 700]


@pytest.mark.parametrize("numel", [1, 3, 4])
def test_few_row_dense_gemm(numel):
    """One dense group of at most 4 rows (the decode shared expert): the
    weight-streaming few-row kernel, K with and without a partial unrolled
    block (7168 = 28 blocks of 256; 2176 = 8 blocks + 2 steps)."""
    d = dev()
    for K in (7168, 2176):
        key = moe_synth.tensor_key(78, numel, K)
        x = moe_synth.normal_bf16(key, (numel, K), 1.0, d)
        wgu = moe_synth.normal_bf16(key + 1, (2 * 256, K), K ** -0.5, d)
        wd = moe_synth.normal_bf16(key + 2, (K, 256), 256 ** -0.5, d)
        one, zero = np.array([numel], np.int32), np.array([0], np.int32)
        gu = mx.grouped_gemm_gate_up(x, wgu, None, 128, 128, fuse_swiglu=False)
        assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu)[None], one, zero), f"gate_up K={K}")
        h = mx.grouped_gemm_gate_up(x, wgu, None, 128, 128, fuse_swiglu=True)
        assert np.array_equal(bits(h), oracle.swiglu(bits(gu), 256))
        y = mx.grouped_gemm_down(h, wd, None, 128, 128)
        assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd)[None], one, zero), f"down K={K}")


@pytest.mark.parametrize("numel", [5, 17, 32])
def test_skinny_dense_gemm(numel):
    """One dense group of 5..32 rows (a shared expert at a decode batch): the
    K-split skinny kernel with K of one step (seven of eight waves idle), of
    uneven splits (3 and 34 steps over 8 waves) and of 112 steps; gate_up
    (K = H) fused and unfused and down (K = F) against the oracle."""
    d = dev()
    for H, F, Hd in ((64, 64, 256), (2176, 192, 2176), (7168, 2176, 7168)):
        key = moe_synth.tensor_key(89, numel, H)
        x = moe_synth.normal_bf16(key, (numel, H), 1.0, d)
        wgu = moe_synth.normal_bf16(key + 1, (2 * F, H), H ** -0.5, d)
        wd = moe_synth.normal_bf16(key + 2, (Hd, F), F ** -0.5, d)
        one, zero = np.array([numel], np.int32), np.array([0], np.int32)
        gu = mx.grouped_gemm_gate_up(x, wgu, None, 128, 128, fuse_swiglu=False)
        assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu)[None], one, zero), f"gate_up H={H}")
        h = mx.grouped_gemm_gate_up(x, wgu, None, 128, 128, fuse_swiglu=True)
        assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
        y = mx.grouped_gemm_down(h, wd, None, 128, 128)
        assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd)[None], one, zero), f"down F={F}")


@pytest.mark.parametrize("layout", ["spread", "last"])
def test_few_row_grouped_gemm(layout):
    """A grouped launch with numel <= E / 10 rows (one decode token's top-k
    over many experts): mostly empty experts, single rows, and one expert
    with 9 rows (more than one pass of the kernel's row batch); "last" puts
    the rows in the highest experts (the expert scan's second 64-wide
    chunk and beyond)."""
    d = dev()
    E, H, F = 160, 256, 384
    sizes = np.zeros(E, np.int64)
    hot = [5, 17, 63, 64, 100, 130, 159] if layout == "spread" else [153, 154, 155, 156, 157, 158, 159]
    for e in hot:
        sizes[e] = 1
    sizes[hot[2]] = 9
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)[:, None]
    assert ids_np.shape[0] * 10 <= E
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    T = ids_np.shape[0]
    key = moe_synth.tensor_key(80, T)
    xp = moe_synth.normal_bf16(key, (T, H), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, H), H ** -0.5, d)
    wd = moe_synth.normal_bf16(key + 2, (E, H, F), F ** -0.5, d)
    gu = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, fuse_swiglu=False)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(xp), bits(wgu), gs, go), "few-row gate_up")
    h = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, fuse_swiglu=True)
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
    y = mx.grouped_gemm_down(h, wd, tb, 128, 128)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd), gs, go), "few-row down")


@pytest.mark.parametrize("fused", [True, False])
def test_grouped_gemm_wide_expert_groups(fused):
    """16 column tiles (the expert-grouped tile order of the 256-row kernel):
    experts of 0 .. 9 row tiles, so blocks of 1, 2 and 4 row tiles and
    left-over row tiles all occur; every output against the oracle."""
    d = dev()
    sizes = [0, 1, 127, 128, 129, 255, 256, 257, 700, 1300, 2100, 513, 1025]
    E, H, F = len(sizes), 128, 2048
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids_np = ids_np[np.random.default_rng(11).permutation(ids_np.size)][:, None]
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    T = ids_np.shape[0]
    key = moe_synth.tensor_key(79, int(fused))
    xp = moe_synth.normal_bf16(key, (T, H), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, H), H ** -0.5, d)
    gu_ref = oracle.grouped_gemm(bits(xp), bits(wgu), gs, go)
    if fused:
        h = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, fuse_swiglu=True)
        assert np.array_equal(bits(h), oracle.swiglu(bits(mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, False)), F))
        assert_bf16_close(bits(mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, False)), gu_ref, "gate_up (16 col tiles)")
    else:
        wd = moe_synth.normal_bf16(key + 2, (E, 4096, H), H ** -0.5, d)
        y = mx.grouped_gemm_down(xp, wd, tb, 128, 128)
        assert_bf16_close(bits(y), oracle.grouped_gemm(bits(xp), bits(wd), gs, go), "down (16 col tiles)")


def test_wide_persistent_claims_repeat_streams_graph():
    """The 256-row kernel runs persistent (one workgroup per CU claiming
    tiles from per-stream counters that each launch returns to zero) when its
    tile list outnumbers the CUs. Outputs pre-filled with NaN bits so a
    skipped tile shows: the first call against the oracle, then the same
    bytes from repeated calls, from calls of another shape in between, from
    two streams at once and from three replays of a captured graph."""
    d = dev()
    sizes = [0, 1, 127, 128, 129, 255, 256, 257, 700, 1300, 2100, 513, 1025]
    E, H, F = len(sizes), 128, 2048
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids_np = ids_np[np.random.default_rng(12).permutation(ids_np.size)][:, None]
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    T = ids_np.shape[0]
    key = moe_synth.tensor_key(78, 0)
    xp = moe_synth.normal_bf16(key, (T, H), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, H), H ** -0.5, d)
    # a second shape between the calls: 40 experts of 0 .. 600 rows, 8 column
    # tiles (the fixed tile groups), also above one tile per CU
    sizes_o = np.random.default_rng(13).integers(0, 601, 40)
    ids_o = np.repeat(np.arange(40, dtype=np.int32), sizes_o)[:, None]
    tbo = mx.moe_align(_t(ids_o, d), 40, 128, 128)
    xo = moe_synth.normal_bf16(key + 2, (ids_o.shape[0], 256), 1.0, d)
    wo = moe_synth.normal_bf16(key + 3, (40, 2048, 256), 256 ** -0.5, d)
    gso, goo = host(tbo["group_sizes"]), host(tbo["group_offsets"])

    def nan_like(n, cols):
        return torch.full((n, cols), -1, dtype=torch.int16, device=d).view(torch.bfloat16)

    def run(out, stream=None):
        out.view(torch.int16).fill_(-1)
        if stream is None:
            return mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, True, out)
        with torch.cuda.stream(stream):
            return mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, True, out)

    h1 = run(nan_like(T, F))
    gu = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, False)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(xp), bits(wgu), gs, go), "gate_up")
    assert np.array_equal(bits(h1), oracle.swiglu(bits(gu), F))
    gu_o = mx.grouped_gemm_gate_up(xo, wo, tbo, 128, 128, False)
    assert_bf16_close(bits(gu_o), oracle.grouped_gemm(bits(xo), bits(wo), gso, goo), "gate_up (40 experts)")
    ref_other = mx.grouped_gemm_gate_up(xo, wo, tbo, 128, 128, True)
    assert np.array_equal(bits(ref_other), oracle.swiglu(bits(gu_o), 1024))
    for i in range(3):
        o = mx.grouped_gemm_gate_up(xo, wo, tbo, 128, 128, True)
        assert torch.equal(o, ref_other), f"other shape, call {i}"
        assert torch.equal(run(nan_like(T, F)), h1), f"repeat {i}"
    s1, s2 = torch.cuda.Stream(d), torch.cuda.Stream(d)
    s1.wait_stream(torch.cuda.current_stream(d))
    s2.wait_stream(torch.cuda.current_stream(d))
    outs = [(nan_like(T, F), s1), (nan_like(T, F), s2), (nan_like(T, F), s1), (nan_like(T, F), s2)]
    for o, s in outs:
        run(o, s)
    torch.cuda.synchronize()
    for i, (o, _) in enumerate(outs):
        assert torch.equal(o, h1), f"two streams, output {i}"
    g_out = nan_like(T, F)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, True, g_out)
    for i in range(3):
        g_out.view(torch.int16).fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out, h1), f"graph replay {i}"
        assert torch.equal(run(nan_like(T, F)), h1), f"eager after replay {i}"
    say("persistent wide kernel: repeats, two streams and graph replays identical")


def test_wide_persistent_more_streams_than_claim_slots():
    """The library keeps claim counters for 64 streams; calls on later streams
    take the one-workgroup-per-tile kernel. 72 new streams (past the 64 slots
    whatever this process used before), each call's output pre-filled with NaN
    bits: every output equal to the first call's bytes, whichever kernel ran."""
    d = dev()
    sizes = np.random.default_rng(14).integers(0, 601, 40)
    ids = np.repeat(np.arange(40, dtype=np.int32), sizes)[:, None]
    tb = mx.moe_align(_t(ids, d), 40, 128, 128)
    key = moe_synth.tensor_key(77, 0)
    x = moe_synth.normal_bf16(key, (ids.shape[0], 256), 1.0, d)
    w = moe_synth.normal_bf16(key + 1, (40, 2048, 256), 256 ** -0.5, d)
    ref = mx.grouped_gemm_gate_up(x, w, tb, 128, 128, True)
    streams = [torch.cuda.Stream(d) for _ in range(72)]
    outs = []
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(d))
        o = torch.full_like(ref.view(torch.int16), -1).view(torch.bfloat16)
        s.wait_stream(torch.cuda.current_stream(d))
        with torch.cuda.stream(s):
            mx.grouped_gemm_gate_up(x, w, tb, 128, 128, True, o)
        outs.append(o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref), f"stream {i}"


@pytest.mark.parametrize("case", ["700_experts", "dense"])
def test_wide_persistent_against_oracle(case):
    """The persistent form on shapes the forwards do not reach: 700 experts of
    100-200 rows (the tile count scans the group sizes in several 512-expert
    batches; two K steps), and one dense group of 65536 rows (no tables). Fused
    and unfused, outputs pre-filled with NaN bits, against the oracle."""
    d = dev()
    key = moe_synth.tensor_key(76, 0 if case == "dense" else 1)
    if case == "dense":
        E, H, F, n = 1, 256, 256, 65536
        tb = None
        x = moe_synth.normal_bf16(key, (n, H), 1.0, d)
        w = moe_synth.normal_bf16(key + 1, (2 * F, H), H ** -0.5, d)
        gs, go = np.array([n], dtype=np.int32), np.array([0], dtype=np.int32)
        w3 = w.view(1, 2 * F, H)
    else:
        E, H, F = 700, 128, 128
        sizes = np.random.default_rng(15).integers(100, 201, E)
        ids = np.repeat(np.arange(E, dtype=np.int32), sizes)
        ids = ids[np.random.default_rng(16).permutation(ids.size)][:, None]
        tb = mx.moe_align(_t(ids, d), E, 128, 128)
        gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
        n = ids.shape[0]
        x = moe_synth.normal_bf16(key, (n, H), 1.0, d)
        w = moe_synth.normal_bf16(key + 1, (E, 2 * F, H), H ** -0.5, d)
        w3 = w
    gu = torch.full((n, 2 * F), -1, dtype=torch.int16, device=d).view(torch.bfloat16)
    mx.grouped_gemm_gate_up(x, w, tb, 128, 128, False, gu)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(w3), gs, go), f"gate_up ({case})")
    h = torch.full((n, F), -1, dtype=torch.int16, device=d).view(torch.bfloat16)
    mx.grouped_gemm_gate_up(x, w, tb, 128, 128, True, h)
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))


@pytest.mark.parametrize("K", [768, 192])
def test_down_column_tile_pairs(K):
    """Unfused grouped launches of short K whose experts average at most 64
    rows give each workgroup two adjacent 256-column tiles: one continued
    ring for the tiles of at most 64 rows when K / 64 is a multiple of the
    ring depth (K = 768), else the two tiles in turn (K = 192, and the
    experts of 100 and 300 rows). Output pre-filled with NaN bits, against
    the oracle."""
    d = dev()
    E, H = 40, 512
    sizes = np.random.default_rng(17).integers(0, 41, E)
    sizes[3], sizes[7], sizes[11] = 100, 300, 64
    ids = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids = ids[np.random.default_rng(18).permutation(ids.size)][:, None]
    assert ids.shape[0] <= 64 * E
    tb = mx.moe_align(_t(ids, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    key = moe_synth.tensor_key(75, K)
    h = moe_synth.normal_bf16(key, (ids.shape[0], K), 1.0, d)
    wd = moe_synth.normal_bf16(key + 1, (E, H, K), K ** -0.5, d)
    y = torch.full((ids.shape[0], H), -1, dtype=torch.int16, device=d).view(torch.bfloat16)
    mx.grouped_gemm_down(h, wd, tb, 128, 128, y)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd), gs, go), f"down K={K}")


@pytest.mark.parametrize("n_out", [4096, 256])
def test_grouped_gemm_more_than_512_experts(n_out):
    """700 experts: the tile search loads the group sizes 512 at a time, so the
    experts past 512 (among them experts of 1..9 row tiles) are found in its
    second pass. n_out = 4096 takes the expert-aware tile order (16 column
    tiles), 256 the fixed groups; gate_up (fused and not) and down against the
    oracle."""
    d = dev()
    say("more than 512 experts", n_out)
    rng = np.random.default_rng(12)
    E = 700
    sizes = (rng.integers(1, 200, E) * (rng.random(E) < 0.35)).astype(np.int64)
    for e, n in ((3, 600), (513, 1), (515, 257), (600, 2300), (650, 700), (699, 129)):
        sizes[e] = n
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids_np = ids_np[rng.permutation(ids_np.size)][:, None]
    T, K = ids_np.shape[0], 64
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    assert list(gs) == list(sizes)
    key = moe_synth.tensor_key(87, n_out)
    x = moe_synth.normal_bf16(key, (T, K), 1.0, d)
    F = n_out // 2
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, K), K ** -0.5, d)
    gu = mx.grouped_gemm_gate_up(x, wgu, tb, 128, 128, fuse_swiglu=False)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu), gs, go), f"gate_up E=700 2F={2 * F}")
    h = mx.grouped_gemm_gate_up(x, wgu, tb, 128, 128, fuse_swiglu=True)
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
    wd = moe_synth.normal_bf16(key + 2, (E, n_out, K), K ** -0.5, d)
    y = mx.grouped_gemm_down(x, wd, tb, 128, 128)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(x), bits(wd), gs, go), f"down E=700 H={n_out}")


@pytest.mark.parametrize("K", [64, 192, 448])
def test_grouped_gemm_small_expert_tiles(K):
    """Tiles of at most 32 valid rows inside a 256-row-kernel launch (experts
    of 1 .. 33 rows, and the last rows of 257 / 289-row experts) beside
    full and half tiles; K of 1, 3 and 7 steps of 64 (the half tiles split
    their K sub-steps between two wave rows). gate_up with H = K, down with
    F = K, fused and unfused, against the oracle."""
    d = dev()
    say("small expert tiles", K)
    sizes = [1, 2, 5, 16, 31, 32, 33, 0, 600, 257, 289, 3, 2000]
    E = len(sizes)
    assert sum(sizes) >= 128 * E                 # the 256-row kernel's launch rule
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids_np = ids_np[np.random.default_rng(K).permutation(ids_np.size)][:, None]
    T = ids_np.shape[0]
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    key = moe_synth.tensor_key(84, K)
    F, H = 128, 256
    x = moe_synth.normal_bf16(key, (T, K), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, K), K ** -0.5, d)
    gu = mx.grouped_gemm_gate_up(x, wgu, tb, 128, 128, fuse_swiglu=False)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu), gs, go), f"gate_up K={K}")
    h = mx.grouped_gemm_gate_up(x, wgu, tb, 128, 128, fuse_swiglu=True)
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
    wd = moe_synth.normal_bf16(key + 2, (E, H, K), K ** -0.5, d)
    y = mx.grouped_gemm_down(x, wd, tb, 128, 128)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(x), bits(wd), gs, go), f"down K={K}")


@pytest.mark.parametrize("K", [2048, 4096])
def test_k_rotation_4k_rows(K):
    """Rows a multiple of 4 KiB long (K = 2048, 4096): the 256-row kernel's
    small-row tiles, the few-row kernel and the skinny kernel walk K from a
    per-expert (or per-column-tile) start and wrap around. 48 experts of 1 ..
    129 rows (their starts cover all 32 or 64 K blocks; 64/65- and
    128/129-row tiles; empty experts) and a 300-row expert (a full tile, not
    rotated, and a rotated 44-row one); 8 single-row experts among 160 (the
    few-row kernel); dense groups of 3 and 20 rows (few-row and skinny
    kernels). gate_up (H = K) fused and unfused, and down (F = K), against
    the oracle."""
    d = dev()
    say("K rotation", K)
    F, Hd = 128, 256
    rng = np.random.default_rng(K + 1)

    def check(x, tb, gs, go, key, label):
        E = len(gs)
        wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, K), K ** -0.5, d)
        wd = moe_synth.normal_bf16(key + 2, (E, Hd, K), K ** -0.5, d)
        if tb is None:
            wgu, wd = wgu[0], wd[0]
        gu = mx.grouped_gemm_gate_up(x, wgu, tb, 128, 128, fuse_swiglu=False)
        wgu3, wd3 = (wgu[None], wd[None]) if tb is None else (wgu, wd)
        assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu3), gs, go), f"{label} gate_up K={K}")
        h = mx.grouped_gemm_gate_up(x, wgu, tb, 128, 128, fuse_swiglu=True)
        assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F)), label
        y = mx.grouped_gemm_down(x, wd, tb, 128, 128)
        assert_bf16_close(bits(y), oracle.grouped_gemm(bits(x), bits(wd3), gs, go), f"{label} down K={K}")

    # small-row tiles of the 256-row kernel
    E = 49
    sizes = rng.integers(1, 130, E)
    sizes[[3, 11]] = 0
    sizes[[5, 6, 7, 8]] = [64, 65, 128, 129]
    sizes[40] = 300
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids_np = ids_np[rng.permutation(ids_np.size)][:, None]
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    assert list(gs) == list(sizes)
    key = moe_synth.tensor_key(91, K)
    check(moe_synth.normal_bf16(key, (ids_np.shape[0], K), 1.0, d), tb, gs, go, key, "small tiles")
    # few-row kernel: one row in each of 8 experts among 160
    E = 160
    sizes = np.zeros(E, np.int64)
    sizes[[2, 33, 70, 101, 127, 140, 150, 159]] = 1
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)[:, None]
    assert ids_np.shape[0] * 10 <= E
    tb = mx.moe_align(_t(ids_np, d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    key = moe_synth.tensor_key(92, K)
    check(moe_synth.normal_bf16(key, (ids_np.shape[0], K), 1.0, d), tb, gs, go, key, "few-row grouped")
    # dense groups: few-row (3 rows) and skinny (20 rows) kernels
    for numel in (3, 20):
        key = moe_synth.tensor_key(93, K, numel)
        one, zero = np.array([numel], np.int32), np.array([0], np.int32)
        check(moe_synth.normal_bf16(key, (numel, K), 1.0, d), None, one, zero, key, f"dense {numel} rows")


@pytest.mark.parametrize("H,F,extra_empty", [(256, 256, 0), (512, 384, 0), (256, 256, 20)])
def test_grouped_gemm_expert_size_edges(H, F, extra_empty):
    """extra_empty appends empty experts; with 20 of them the rows per expert
    average under one 128-row block, which selects the 128-row tile kernel
    instead of the 256-row one."""
    d = dev()
    say("gemm edges", H, F, extra_empty)
    sizes = EDGE_SIZES + [0] * extra_empty
    E = len(sizes)
    ids_np = np.repeat(np.arange(E, dtype=np.int32), sizes)
    ids_np = ids_np[np.random.default_rng(7).permutation(ids_np.size)][:, None]
    T = ids_np.shape[0]
    ids = _t(ids_np, d)
    tb = mx.moe_align(ids, E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    assert list(gs) == sizes
    key = moe_synth.tensor_key(71, H)
    xp = moe_synth.normal_bf16(key, (T, H), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (E, 2 * F, H), H ** -0.5, d)
    wd = moe_synth.normal_bf16(key + 2, (E, H, F), F ** -0.5, d)
    gu = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, fuse_swiglu=False)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(xp), bits(wgu), gs, go), "gate_up")
    h = mx.grouped_gemm_gate_up(xp, wgu, tb, 128, 128, fuse_swiglu=True)
    assert torch.equal(h, mx.swiglu(gu))
    y = mx.grouped_gemm_down(h, wd, tb, 128, 128)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd), gs, go), "down")
    # same inputs again: bitwise repeatable
    assert torch.equal(mx.grouped_gemm_down(h, wd, tb, 128, 128), y)


@pytest.mark.parametrize("numel", [1, 129, 300, 4224])
def test_dense_gemm_wide_shapes(numel):
    d = dev()
    H, F = 256, 256
    key = moe_synth.tensor_key(72, numel)
    x = moe_synth.normal_bf16(key, (numel, H), 1.0, d)
    wgu = moe_synth.normal_bf16(key + 1, (2 * F, H), H ** -0.5, d)
    wd = moe_synth.normal_bf16(key + 2, (H, F), F ** -0.5, d)
    one, zero = np.array([numel], np.int32), np.array([0], np.int32)
    gu = mx.grouped_gemm_gate_up(x, wgu, None, 128, 128, fuse_swiglu=False)
    assert_bf16_close(bits(gu), oracle.grouped_gemm(bits(x), bits(wgu)[None], one, zero), "dense gate_up")
    h = mx.grouped_gemm_gate_up(x, wgu, None, 128, 128, fuse_swiglu=True)
    assert torch.equal(h, mx.swiglu(gu))
    y = mx.grouped_gemm_down(h, wd, None, 128, 128)
    assert_bf16_close(bits(y), oracle.grouped_gemm(bits(h), bits(wd)[None], one, zero), "dense down")


# --------------------------------------------------------------- swiglu --

def test_swiglu_bit_exact_including_extremes():
    d = dev()
    M, F = 257, 256
    x = bits(moe_synth.normal_bf16(moe_synth.tensor_key(71), (M, 2 * F), 3.0, "cpu"))
    specials = nm.to_bf16(np.array([0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 90.0, -90.0, 1e30, -1e30,
                                    1e-38, 2.0 ** -133, 87.0, -87.0, 0.5, -0.5]))
    x[0, :len(specials)] = specials
    x[1, F:F + len(specials)] = specials
    x[2, :len(specials)] = specials[::-1]
    x[2, F:F + len(specials)] = specials
    h = mx.swiglu(_bf16_dev(x, d))
    assert np.array_equal(bits(h), oracle.swiglu(x, F))


# ------------------------------------------------ aligned grouped GEMM --

def _aligned_tables(E, M, d):
    T = E * M
    ids = torch.arange(E, dtype=torch.int32, device=d).repeat_interleave(M).view(T, 1)
    tb = mx.moe_align(ids, E, 128, 128)
    assert np.array_equal(host(tb["group_sizes"]), np.full(E, M))
    return tb


@pytest.mark.parametrize("E,M,N,K", [(3, 512, 256, 384), (2, 1024, 640, 192), (5, 256, 128, 128)])
def test_aligned_gemm_small(E, M, N, K):
    """Aligned groups (every group a whole number of 256-row tiles), every output."""
    d = dev()
    key = moe_synth.tensor_key(77, E, M, N, K)
    a = moe_synth.normal_bf16(key, (E * M, K), 1.0, d)
    w = moe_synth.normal_bf16(key + 1, (E, N, K), K ** -0.5, d)
    tb = _aligned_tables(E, M, d)
    y = mx.grouped_gemm_down(a, w, tb, 128, 128)
    ref = oracle.grouped_gemm(bits(a), bits(w), np.full(E, M), np.arange(E) * M)
    assert_bf16_close(bits(y), ref, "aligned grouped GEMM")


@pytest.mark.parametrize("name", ["glm5_up_t32768", "glm5_down_t262144", "llama4_128e_down_t131072",
                                  "qwen3.5_397b_down_t52429"])
def test_aligned_gemm_table_shape_sampled_rows(name):
    """A table shape at full size, launched as the benchmark launches it: every
    output column of sampled rows (tile edges and random rows) in sampled
    groups (first, last, random), against the oracle."""
    d = dev()
    case = moe_synth.GEMM_CASES[name]
    say("aligned gemm", name)
    a = moe_synth.gemm_a(case, d)
    w = moe_synth.gemm_w(case, d)
    tb = _aligned_tables(case.E, case.M, d)
    y = mx.grouped_gemm_down(a, w, tb, 128, 128)
    rng = np.random.default_rng(case.cid)
    groups = sorted({0, case.E - 1, *rng.choice(case.E, 2, replace=False).tolist()})
    rows = sorted({0, 127, 128, 255, 256, case.M - 1, *rng.choice(case.M, 4, replace=False).tolist()})
    for e in groups:
        r = torch.as_tensor(e * case.M + np.asarray(rows), device=d)
        ref = oracle.grouped_gemm(bits(a[r]), bits(w[e:e + 1]), np.array([len(rows)]), np.array([0]))
        assert_bf16_close(bits(y[r]), ref, f"{name} group {e}")


# ------------------------------------------------------------- unpermute --

@pytest.mark.parametrize("name", ["tiny", "qwen3_decode"])
def test_unpermute_and_linearity(name):
    d = dev()
    cfg = moe_synth.CONFIGS[name]
    T, k, H = cfg.T, cfg.top_k, cfg.H
    y = moe_synth.normal_bf16(moe_synth.tensor_key(72, cfg.cid), (T * k, H), 0.5, d)
    ids, w = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), k)
    tb = mx.moe_align(ids, cfg.E, cfg.padding_m, cfg.block_m)
    add = moe_synth.normal_bf16(moe_synth.tensor_key(73, cfg.cid), (T, H), 0.5, d)
    p2r = host(tb["pair_to_row"])
    for rsf in (1.0, 2.827):
        o = mx.moe_unpermute(y, tb["pair_to_row"], w, rsf)
        assert_bf16_close(bits(o), oracle.unpermute(bits(y), p2r, host(w), k, rsf), f"unpermute rsf={rsf}")
        o = mx.moe_unpermute(y, tb["pair_to_row"], w, rsf, addend=add)
        assert_bf16_close(bits(o), oracle.unpermute(bits(y), p2r, host(w), k, rsf, bits(add)), "unpermute+addend")
    o1 = nm.bf16_to_f64(bits(mx.moe_unpermute(y, tb["pair_to_row"], w, 1.0)))
    for rsf in (2.0, 0.5):
        o = nm.bf16_to_f64(bits(mx.moe_unpermute(y, tb["pair_to_row"], w, rsf)))
        assert np.array_equal(o, rsf * o1)


@pytest.mark.parametrize("T,k,H,E", [(7, 3, 200, 5), (37, 16, 64, 40), (5, 2, 16392, 4), (301, 1, 2056, 3),
                                     (3, 5, 1024, 9)])
def test_unpermute_ragged_shapes(T, k, H, E):
    """Rows that end inside a wave's 128-chunk item, several items per row, a
    token count that leaves the last workgroup's waves partly idle, every top_k
    template (1..16), with and without the addend."""
    d = dev()
    rng = np.random.default_rng(T * 7 + H)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tb = mx.moe_align(_t(ids, d), E, 16, 16)
    y = moe_synth.normal_bf16(moe_synth.tensor_key(75, H, k), (T * k, H), 0.5, d)
    add = moe_synth.normal_bf16(moe_synth.tensor_key(76, H, k), (T, H), 0.5, d)
    w = torch.as_tensor(rng.uniform(0.0, 1.0, (T, k)).astype(np.float32), device=d)
    p2r = host(tb["pair_to_row"])
    o = mx.moe_unpermute(y, tb["pair_to_row"], w, 1.5)
    assert_bf16_close(bits(o), oracle.unpermute(bits(y), p2r, host(w), k, 1.5), "unpermute")
    o = mx.moe_unpermute(y, tb["pair_to_row"], w, 1.5, addend=add)
    assert_bf16_close(bits(o), oracle.unpermute(bits(y), p2r, host(w), k, 1.5, bits(add)), "unpermute+addend")


# -------------------------------------------------------------- quantizer --

def _quant_compare(x_bits, F, q, rows=None):
    ref = oracle.swiglu_quant_fp8(x_bits, F)
    M = x_bits.shape[0]
    if rows is None:
        assert np.array_equal(host(q["q_row"]), ref["q_row"])
        assert np.array_equal(host(q["s_row"]).view(np.uint32), ref["s_row"].view(np.uint32))
        assert np.array_equal(host(q["q_t"]), ref["q_t"])
        assert np.array_equal(host(q["s_t"]).view(np.uint32), ref["s_t"].view(np.uint32))
    else:
        r0, r1 = rows
        mb = r0 // 128
        assert np.array_equal(host(q["q_row"][r0:r1]), ref["q_row"])
        assert np.array_equal(host(q["s_row"][r0:r1]).view(np.uint32), ref["s_row"].view(np.uint32))
        assert np.array_equal(host(q["q_t"][:, r0:r0 + ref["q_t"].shape[1]]), ref["q_t"])
        assert np.array_equal(host(q["s_t"][:, mb:mb + ref["s_t"].shape[1]]).view(np.uint32),
                              ref["s_t"].view(np.uint32))
    return M


@pytest.mark.parametrize("M", moe_synth.QUANT_EDGE_M)
def test_swiglu_quant_edge_sizes(M):
    d = dev()
    F = moe_synth.QUANT_CONFIG.F
    x = moe_synth.quant_input(M, F, d)
    q = mx.swiglu_quant_fp8(x)
    assert q["q_t"].shape == (F, -(-M // 128) * 128)
    if M:
        _quant_compare(bits(x), F, q)


def test_swiglu_quant_matches_unfused_pair():
    d = dev()
    M, F = 300, 512
    x = moe_synth.quant_input(M, F, d)
    q = mx.swiglu_quant_fp8(x)
    h = bits(mx.swiglu(x))
    ref = oracle.quant_fp8(h)
    for key in ("q_row", "s_row", "q_t", "s_t"):
        assert np.array_equal(host(q[key]).view(np.uint8), ref[key].view(np.uint8)), key


def test_swiglu_quant_every_bf16_code():
    """gate = 64 makes silu(gate) exactly 64, up = v/64 makes h = v for every bf16 v in [-448, 448];
    448 in each row pins the row scale to 1, so the codes are the plain e4m3 encodings."""
    d = dev()
    f = nm.bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    vals = f[np.isfinite(f) & (np.abs(f) <= 448.0) & ((np.abs(f) >= 2.0 ** -100) | (f == 0))]
    per = 127
    n_rows = -(-vals.size // per)
    F = 128
    h = np.zeros((n_rows, F), np.float64)
    h[:, 0] = 448.0
    flat = np.zeros(n_rows * per)
    flat[:vals.size] = vals
    h[:, 1:] = flat.reshape(n_rows, per)
    gate = np.full((n_rows, F), 64.0)
    x = np.concatenate([nm.to_bf16(gate), nm.to_bf16(h / 64.0)], axis=1)
    assert np.array_equal(nm.bf16_to_f64(x[:, F:]) * 64.0, h)   # exact construction
    q = mx.swiglu_quant_fp8(_bf16_dev(x, d))
    assert np.all(host(q["s_row"]) == 1.0)
    assert np.array_equal(host(q["q_row"]), nm.e4m3_encode(h))
    _quant_compare(x, F, q)


def test_swiglu_quant_full_size_sampled_blocks():
    d = dev()
    M, F = moe_synth.QUANT_CONFIG.M, moe_synth.QUANT_CONFIG.F
    x = moe_synth.quant_input(M, F, d)
    q = mx.swiglu_quant_fp8(x)
    for r0 in (0, 128 * 97, M - 128):
        _quant_compare(bits(x[r0:r0 + 128]), F, q, rows=(r0, r0 + 128))


# ------------------------------------------------- block-scaled FP8 GEMM --

def _fp8_case(sizes, N, K, key, d, shuffle=True):
    """Routing with the given per-expert row counts, bf16 activations h and
    weights w; returns (tables, h, w, group sizes, offsets)."""
    E = len(sizes)
    ids = np.repeat(np.arange(E, dtype=np.int32), sizes)
    if shuffle:
        ids = ids[np.random.default_rng(key).permutation(ids.size)]
    tb = mx.moe_align(_t(ids[:, None], d), E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    assert list(gs) == list(sizes)
    numel = int(sum(sizes))
    h = moe_synth.normal_bf16(moe_synth.tensor_key(key, numel, K), (numel, K), 1.0, d)
    w = moe_synth.normal_bf16(moe_synth.tensor_key(key + 1, N, K), (E, N, K), K ** -0.5, d)
    return tb, h, w, gs, go


def test_fp8_block_quant_weights_bit_exact():
    d = dev()
    w = moe_synth.normal_bf16(moe_synth.tensor_key(95), (3, 256, 384), 0.05, d)
    w[1, :128, 128:256] = 0.0                      # an all-zero block
    q = mx.fp8_block_quant_weights(w)
    for e in range(3):
        ref = oracle.block_quant_fp8(bits(w[e]))
        assert np.array_equal(host(q["q"][e]), ref["q"]), e
        assert np.array_equal(host(q["s"][e]).view(np.uint32), ref["s"].view(np.uint32)), e
    assert not q["q"][1, :128, 128:256].any() and q["s"][1, 0, 1].item() == 0.0


@pytest.mark.parametrize("N,K,extra_empty", [(256, 256, 0), (384, 512, 3), (512, 384, 2), (768, 128, 0)])
def test_grouped_gemm_fp8_expert_size_edges(N, K, extra_empty):
    """Expert sizes around the 128-row block (0, 1, 127..129, 255..257, ...),
    empty experts, every output against the oracle on the oracle's own codes;
    the GPU's codes equal the oracle's bit for bit; two to six 128-column
    tiles, K of one to four 128-wide steps."""
    d = dev()
    sizes = EDGE_SIZES + [0] * extra_empty
    tb, h, w, gs, go = _fp8_case(sizes, N, K, 96 + extra_empty, d)
    qa = mx.tile_quant_fp8(h, None)
    qw = mx.fp8_block_quant_weights(w)
    y = mx.grouped_gemm_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], tb, 128)
    ra = oracle.quant_fp8(bits(h))
    rw = [oracle.block_quant_fp8(bits(w[e])) for e in range(len(sizes))]
    assert np.array_equal(host(qa["q_row"]), ra["q_row"]) and np.array_equal(host(qa["s_row"]), ra["s_row"])
    rq = np.stack([r["q"] for r in rw]); rs = np.stack([r["s"] for r in rw])
    assert np.array_equal(host(qw["q"]), rq) and np.array_equal(host(qw["s"]), rs)
    ref = oracle.grouped_gemm_fp8(ra["q_row"], ra["s_row"], rq, rs, gs, go)
    err = assert_bf16_close(bits(y), ref, "fp8 grouped gemm")
    say("  fp8 gemm max abs err", err)


@pytest.mark.parametrize("F,H,extra_empty", [(128, 256, 0), (256, 384, 3)])
def test_grouped_gemm_gate_up_fp8(F, H, extra_empty):
    """Block-scaled FP8 gate_up on expert sizes around the 128-row block:
    unfused against the oracle's product on the oracle's own codes; fused
    equal to swiglu() of the unfused bytes; the same through the gather
    (token codes read via sorted_pair, top_k = 2) as on the permuted codes;
    one dense group."""
    d = dev()
    sizes = EDGE_SIZES + [0] * extra_empty
    tb, x, wgu, gs, go = _fp8_case(sizes, 2 * F, H, 98 + extra_empty, d)
    qa = mx.tile_quant_fp8(x, transposed=False)
    qw = mx.fp8_block_quant_weights(wgu)
    gu = mx.grouped_gemm_gate_up_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], tb, 128, fuse_swiglu=False)
    ra = oracle.quant_fp8(bits(x))
    rw = [oracle.block_quant_fp8(bits(wgu[e])) for e in range(len(sizes))]
    assert np.array_equal(host(qa["q_row"]), ra["q_row"]) and np.array_equal(host(qa["s_row"]), ra["s_row"])
    rq = np.stack([r["q"] for r in rw]); rs = np.stack([r["s"] for r in rw])
    ref = oracle.grouped_gemm_fp8(ra["q_row"], ra["s_row"], rq, rs, gs, go)
    err = assert_bf16_close(bits(gu), ref, "fp8 gate_up")
    say("  fp8 gate_up max abs err", err)
    h = mx.grouped_gemm_gate_up_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], tb, 128)
    assert torch.equal(h, mx.swiglu(gu))
    assert np.array_equal(bits(h), oracle.swiglu(bits(gu), F))
    # gather: T tokens with two slots each; the compact rows are the tokens' codes in sorted_pair order
    # (enough rows per expert for the 256 x 256 kernel)
    T, k = 2000, 2
    rng = np.random.default_rng(F + H)
    ids = np.stack([rng.permutation(len(sizes))[:k] for _ in range(T)]).astype(np.int32)
    tb2 = mx.moe_align(_t(ids, d), len(sizes), 128, 128)
    xt = moe_synth.normal_bf16(moe_synth.tensor_key(99, T, H), (T, H), 1.0, d)
    qt = mx.tile_quant_fp8(xt, transposed=False)
    hg = mx.grouped_gemm_gate_up_fp8(qt["q_row"], qt["s_row"], qw["q"], qw["s"], tb2, 128, top_k=k)
    tok = tb2["sorted_pair"].long() // k
    hc = mx.grouped_gemm_gate_up_fp8(qt["q_row"][tok].contiguous(), qt["s_row"][tok].contiguous(), qw["q"],
                                     qw["s"], tb2, 128)
    assert torch.equal(hg, hc)
    # one dense group
    qd = mx.grouped_gemm_gate_up_fp8(qa["q_row"][:300].contiguous(), qa["s_row"][:300].contiguous(), qw["q"][0],
                                     qw["s"][0], None, 128, fuse_swiglu=False)
    one, zero = np.array([300], np.int32), np.array([0], np.int32)
    refd = oracle.grouped_gemm_fp8(ra["q_row"][:300], ra["s_row"][:300], rq[:1], rs[:1], one, zero)
    assert_bf16_close(bits(qd), refd, "fp8 gate_up dense")


def test_grouped_gemm_fp8_dense_group():
    d = dev()
    M, N, K = 300, 256, 384
    h = moe_synth.normal_bf16(moe_synth.tensor_key(97), (M, K), 1.0, d)
    w = moe_synth.normal_bf16(moe_synth.tensor_key(98), (N, K), K ** -0.5, d)
    qa, qw = mx.tile_quant_fp8(h, None), mx.fp8_block_quant_weights(w)
    y = mx.grouped_gemm_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], None, 128)
    ra, rw = oracle.quant_fp8(bits(h)), oracle.block_quant_fp8(bits(w))
    ref = oracle.grouped_gemm_fp8(ra["q_row"], ra["s_row"], rw["q"][None], rw["s"][None], np.array([M]), np.array([0]))
    assert_bf16_close(bits(y), ref, "fp8 dense")


def test_grouped_gemm_fp8_dsv3_down_sampled_rows():
    """The DeepSeek-V3-shaped routed down projection at full size (numel 32768,
    N = H = 7168, K = F = 2048, 256 experts, Zipf-biased routing): rows of
    sampled experts against the oracle on its own codes."""
    d = dev()
    cfg = moe_synth.CONFIGS["dsv3_prefill"]
    say("fp8 down", cfg.name)
    ids, _ = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), cfg.top_k, expert_bias=moe_synth.expert_bias(cfg, d))
    tb = mx.moe_align(ids, cfg.E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    h = moe_synth.normal_bf16(moe_synth.tensor_key(99), (cfg.numel, cfg.F), 1.0, d)
    wd = moe_synth.w_down(cfg, d)
    qa, qw = mx.tile_quant_fp8(h, None), mx.fp8_block_quant_weights(wd)
    y = mx.grouped_gemm_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], tb, 128)
    active = np.nonzero(gs)[0]
    rng = np.random.default_rng(3)
    for e in sorted({int(active[0]), int(active[-1]), int(np.argmax(gs)), *rng.choice(active, 2).tolist()}):
        o, n = int(go[e]), int(gs[e])
        rows = sorted({0, n - 1, *rng.choice(n, min(n, 6), replace=False).tolist()})
        sel = torch.as_tensor(o + np.asarray(rows), device=d)
        ra = oracle.quant_fp8(bits(h[sel]))
        rw = oracle.block_quant_fp8(bits(wd[e]))
        ref = oracle.grouped_gemm_fp8(ra["q_row"], ra["s_row"], rw["q"][None], rw["s"][None],
                                      np.array([len(rows)]), np.array([0]))
        assert_bf16_close(bits(y[sel]), ref, f"fp8 down expert {e}")


def test_grouped_gemm_gate_up_fp8_dsv3_sampled_rows():
    """The DeepSeek-V3-shaped routed gate_up in FP8 at full size (T = 4096,
    top-8, H = 7168, F = 2048, 256 experts, Zipf-biased routing), reading each
    pair's token codes through sorted_pair, SwiGLU fused: rows of sampled
    experts against the oracle's FP8 product and SwiGLU on its own codes."""
    d = dev()
    cfg = moe_synth.CONFIGS["dsv3_prefill"]
    say("fp8 gate_up", cfg.name)
    ids, _ = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), cfg.top_k, expert_bias=moe_synth.expert_bias(cfg, d))
    tb = mx.moe_align(ids, cfg.E, 128, 128)
    gs, go = host(tb["group_sizes"]), host(tb["group_offsets"])
    sp = host(tb["sorted_pair"])
    hid = moe_synth.hidden(cfg, d)
    wgu = moe_synth.w_gate_up(cfg, d)
    qh, qg = mx.tile_quant_fp8(hid, transposed=False), mx.fp8_block_quant_weights(wgu)
    h = mx.grouped_gemm_gate_up_fp8(qh["q_row"], qh["s_row"], qg["q"], qg["s"], tb, 128, top_k=cfg.top_k)
    active = np.nonzero(gs)[0]
    rng = np.random.default_rng(4)
    for e in sorted({int(active[0]), int(active[-1]), int(np.argmax(gs)), *rng.choice(active, 2).tolist()}):
        o, n = int(go[e]), int(gs[e])
        rows = sorted({0, n - 1, *rng.choice(n, min(n, 6), replace=False).tolist()})
        tok = torch.as_tensor(sp[o + np.asarray(rows)] // cfg.top_k, device=d)
        ra = oracle.quant_fp8(bits(hid[tok]))
        rw = oracle.block_quant_fp8(bits(wgu[e]))
        ref = oracle.grouped_gemm_fp8(ra["q_row"], ra["s_row"], rw["q"][None], rw["s"][None],
                                      np.array([len(rows)]), np.array([0]))
        sel = torch.as_tensor(o + np.asarray(rows), device=d)
        got = bits(h[sel])
        exp = oracle.swiglu(ref, cfg.F)
        # SwiGLU of the bf16 products: compare against the oracle's SwiGLU of its own product
        assert_bf16_close(got, exp, f"fp8 gate_up expert {e}")


# ------------------------------------------- grouped tile quantizer --

def _tq_equal(got, ref, name, rows=None, cols=None, scols=None):
    for k in ("q_row", "s_row"):
        g = host(got[k]) if rows is None else host(got[k][rows[0]:rows[1]])
        assert np.array_equal(g.view(np.uint8 if k == "q_row" else np.uint32),
                              ref[k].view(np.uint8 if k == "q_row" else np.uint32)), (name, k)
    qt = host(got["q_t"]) if cols is None else host(got["q_t"][:, cols[0]:cols[1]])
    st = host(got["s_t"]) if scols is None else host(got["s_t"][:, scols[0]:scols[1]])
    assert np.array_equal(qt, ref["q_t"]), (name, "q_t")
    assert np.array_equal(st.view(np.uint32), ref["s_t"].view(np.uint32)), (name, "s_t")


@pytest.mark.parametrize("per_tile", [False, True])
@pytest.mark.parametrize("swiglu", [False, True])
def test_tile_quant_page_group_sizes(per_tile, swiglu):
    """Group sizes [0, 1, 127, 128, 129] with K=6144 (the grouped quantizers'
    test case), at the exact padded width and at the bound width (the columns
    past the groups' total must come back zero), every output byte."""
    d = dev()
    case = dataclasses.replace(moe_synth.GROUPED_QUANT_CASES["quant_groups_0_1_127_128_129_k6144"], swiglu=swiglu)
    sizes = moe_synth.grouped_quant_sizes(case)
    x = moe_synth.grouped_quant_input(case, d)
    h = oracle.swiglu(bits(x), case.K) if swiglu else bits(x)
    trans = "tile" if per_tile else "block"
    gs = _t(sizes, d)
    for m_pad in (640, mx.tile_quant_fp8_m_pad_bound(case.M, case.E)):
        q = mx.tile_quant_fp8(x, gs, per_tile=per_tile, swiglu=swiglu, m_pad=m_pad)
        ref = oracle.quant_fp8_grouped(h, sizes, trans, m_pad=m_pad)
        _tq_equal(q, ref, f"page groups m_pad={m_pad}")


@pytest.mark.parametrize("per_tile", [False, True])
def test_tile_quant_random_groups_and_overwrite(per_tile):
    """Random group sizes (empty groups, tiny groups, several blocks), outputs
    pre-filled with 0xFF / NaN so every byte the contract covers must be written."""
    d = dev()
    rng = np.random.default_rng(90 + per_tile)
    sizes = rng.choice([0, 1, 5, 127, 128, 129, 300, 513], size=11).astype(np.int32)
    M, K = int(sizes.sum()), 256
    x = moe_synth.normal_bf16(moe_synth.tensor_key(91, M, per_tile), (M, K), 1.0, d)
    m_pad = mx.tile_quant_fp8_m_pad_bound(M, len(sizes))
    out = {"q_row": torch.full((M, K), 0xFF, dtype=torch.uint8, device=d),
           "s_row": torch.full((M, K // 128), float("nan"), device=d),
           "q_t": torch.full((K, m_pad), 0xFF, dtype=torch.uint8, device=d),
           "s_t": torch.full(((K if per_tile else K // 128), m_pad // 128), float("nan"), device=d)}
    q = mx.tile_quant_fp8(x, _t(sizes, d), per_tile=per_tile, m_pad=m_pad, out=out)
    ref = oracle.quant_fp8_grouped(bits(x), sizes, "tile" if per_tile else "block", m_pad=m_pad)
    _tq_equal(q, ref, f"random groups {sizes.tolist()}")



@pytest.mark.parametrize("per_tile,swiglu,n_groups,K", [(False, False, 64, 2048), (True, False, 64, 2048),
                                                        (False, True, 64, 2048), (False, False, 400, 256),
                                                        (True, False, 700, 256)])
def test_tile_quant_paired_blocks_overwrite(per_tile, swiglu, n_groups, K):
    """A grouped launch large enough that each workgroup takes two adjacent
    column blocks (over 2048 blocks; the per-tile SwiGLU form stays
    unpaired; the group-size scan loads 512 sizes at a time, so 700 groups
    take two passes of it): random ragged groups, outputs pre-filled so every
    byte the contract covers must be written, including the zero columns of
    the padded tails."""
    d = dev()
    rng = np.random.default_rng(95 + n_groups)
    sizes = rng.choice([0, 1, 5, 127, 128, 129, 300, 513, 1000], size=n_groups).astype(np.int32)
    M = int(sizes.sum())
    m_pad = mx.tile_quant_fp8_m_pad_bound(M, len(sizes))
    assert (m_pad // 128) * (K // 128) >= 2048
    say("paired tile quant", M, K, m_pad, per_tile, swiglu)
    x = moe_synth.normal_bf16(moe_synth.tensor_key(96, M, int(swiglu)), (M, 2 * K if swiglu else K), 1.0, d)
    out = {"q_row": torch.full((M, K), 0xFF, dtype=torch.uint8, device=d),
           "s_row": torch.full((M, K // 128), float("nan"), device=d),
           "q_t": torch.full((K, m_pad), 0xFF, dtype=torch.uint8, device=d),
           "s_t": torch.full((K if per_tile else K // 128, m_pad // 128), float("nan"), device=d)}
    q = mx.tile_quant_fp8(x, _t(sizes, d), per_tile=per_tile, swiglu=swiglu, m_pad=m_pad, out=out)
    h = oracle.swiglu(bits(x), K) if swiglu else bits(x)
    ref = oracle.quant_fp8_grouped(h, sizes, "tile" if per_tile else "block", m_pad=m_pad)
    _tq_equal(q, ref, f"paired blocks per_tile={per_tile} swiglu={swiglu} groups={n_groups}")


def test_tile_quant_ungrouped_equals_swiglu_quant_fp8():
    """One group, block scales, SwiGLU input: the same bytes as swiglu_quant_fp8
    (and as quantizing the unfused SwiGLU output without it)."""
    d = dev()
    for M in (1, 129, 1000):
        x = moe_synth.quant_input(M, 256, d)
        a = mx.swiglu_quant_fp8(x)
        b = mx.tile_quant_fp8(x, None, per_tile=False, swiglu=True)
        c = mx.tile_quant_fp8(mx.swiglu(x), None)
        for k in a:
            assert torch.equal(a[k], b[k]), (M, k)
            assert torch.equal(a[k], c[k]), (M, k, "h")


@pytest.mark.parametrize("M", [1, 127, 300, 4224])
@pytest.mark.parametrize("swiglu", [False, True])
def test_tile_quant_row_only(M, swiglu):
    """q_t = s_t = NULL: the row layout alone, the same bytes as the full call
    (ungrouped and grouped) and as the oracle."""
    d = dev()
    K = 256
    key = moe_synth.tensor_key(87, M, int(swiglu))
    x = moe_synth.normal_bf16(key, (M, 2 * K if swiglu else K), 1.0, d)
    rows = mx.tile_quant_fp8(x, None, swiglu=swiglu, transposed=False)
    assert set(rows) == {"q_row", "s_row"}
    full = mx.tile_quant_fp8(x, None, swiglu=swiglu)
    assert torch.equal(rows["q_row"], full["q_row"]) and torch.equal(rows["s_row"], full["s_row"])
    sizes = np.random.default_rng(M).multinomial(M, np.ones(5) / 5).astype(np.int32)
    grouped = mx.tile_quant_fp8(x, _t(sizes, d), swiglu=swiglu)
    assert torch.equal(rows["q_row"], grouped["q_row"]) and torch.equal(rows["s_row"], grouped["s_row"])
    h = oracle.swiglu(bits(x), K) if swiglu else bits(x)
    ref = oracle.quant_fp8(h)
    assert np.array_equal(host(rows["q_row"]), ref["q_row"]) and np.array_equal(host(rows["s_row"]), ref["s_row"])


def test_tile_quant_zero_rows_zero_fills():
    d = dev()
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=d)
    gs = _t(np.zeros(3, np.int32), d)
    q = mx.tile_quant_fp8(x, gs, per_tile=True, m_pad=384,
                          out={"q_t": torch.full((256, 384), 7, dtype=torch.uint8, device=d),
                               "s_t": torch.full((256, 3), 7.0, device=d)})
    assert not q["q_t"].any() and not q["s_t"].any()


@pytest.mark.parametrize("name,per_tile", [("quant_131072x6144_e256", False), ("quant_131072x6144_e256", True),
                                           ("swiglu_quant_131072x8192_e256", False)])
def test_tile_quant_benchmark_shapes_sampled_groups(name, per_tile):
    """The benchmark shapes at full size, launched as the benchmark launches
    them: the row layout of sampled groups' rows, and their transposed columns
    and scales (each group's part is the oracle run on that group's rows
    alone, at its expanded offset); columns past the total are zero."""
    d = dev()
    case = moe_synth.GROUPED_QUANT_CASES[name]
    say("tile quant", name, per_tile)
    sizes = moe_synth.grouped_quant_sizes(case)
    x = moe_synth.grouped_quant_input(case, d)
    q = mx.tile_quant_fp8(x, _t(sizes, d), per_tile=per_tile, swiglu=case.swiglu)
    starts, total = oracle.expand_128x_starts(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    trans = "tile" if per_tile else "block"
    for g in sorted({0, 1, len(sizes) - 1, *np.random.default_rng(case.cid).choice(len(sizes), 3).tolist()}):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        xb = bits(x[r0:r1])
        h = oracle.swiglu(xb, case.K) if case.swiglu else xb
        ref = oracle.quant_fp8_grouped(h, None, trans)
        w = ref["q_t"].shape[1]
        _tq_equal(q, ref, f"{name} group {g}", rows=(r0, r1), cols=(starts[g], starts[g] + w),
                  scols=(starts[g] // 128, (starts[g] + w) // 128))
    assert not q["q_t"][:, total:].any() and not q["s_t"][:, total // 128:].any()


# ----------------------------------------------------------- end to end --

def _gpu_forward(cfg, inp, fuse=True, **kw):
    return mx.routed_moe_forward(inp["hidden"], inp["logits"], inp["w_gate_up"], inp["w_down"], cfg.top_k,
                                 cfg.rsf, cfg.padding_m, cfg.block_m, inp.get("shared_w_gate_up"),
                                 inp.get("shared_w_down"), fuse_swiglu=fuse, expert_bias=inp.get("bias"),
                                 scoring=cfg.scoring, renormalize=cfg.renormalize, **kw)


@pytest.mark.parametrize("name", ["tiny", "qwen3_decode"])
def test_forward_full_oracle(name):
    d = dev()
    cfg = moe_synth.CONFIGS[name]
    say("forward", name)
    inp = inputs(cfg, d)
    ref = oracle.forward(bits(inp["hidden"]), host(inp["logits"]), bits(inp["w_gate_up"]), bits(inp["w_down"]),
                         cfg.top_k, cfg.rsf, cfg.padding_m, cfg.block_m)
    assert "bias" not in inp and cfg.scoring == "softmax"
    for fuse in (True, False):
        out = _gpu_forward(cfg, inp, fuse)
        err = assert_bf16_close(bits(out), ref["out"], f"{name} out fuse={fuse}")
        say("  out max abs err", err, "fuse", fuse)
        # the permute as its own copy kernel instead of inside gate_up's loads: same bytes
        assert torch.equal(_gpu_forward(cfg, inp, fuse, fuse_permute=False), out)


def test_forward_kimi_k2_single_token():
    """The Kimi-K2-shaped forward at T=1 (decode of one token: 8 of 384 experts,
    one row each, plus the 18432-wide shared expert), every output element
    against the oracle."""
    d = dev()
    cfg = moe_synth.CONFIGS["kimi_k2_t1"]
    say("forward", cfg.name)
    inp = inputs(cfg, d)
    ref = oracle_tokens(cfg, inp, [0])
    side = torch.cuda.Stream(d)
    for fuse in (True, False):
        out = _gpu_forward(cfg, inp, fuse)
        err = assert_bf16_close(bits(out), ref["out"], f"kimi T=1 out fuse={fuse}")
        say("  out max abs err", err, "fuse", fuse)
        assert torch.equal(_gpu_forward(cfg, inp, fuse, shared_stream=side), out)


SHARED_SMALL = moe_synth.MoEConfig(85, "shared_small", T=64, H=256, F=128, E=16, top_k=4, padding_m=128,
                                   block_m=128, shared_F=384, scoring="sigmoid")


@pytest.mark.parametrize("name,side,fp8", [("qwen3_decode", False, False), ("qwen3_prefill", False, False),
                                           ("shared_small", False, False), ("shared_small", True, False),
                                           ("shared_small", True, True)])
def test_forward_graph_replay(name, side, fp8):
    """The forward captured as a HIP graph (with the shared expert forked onto
    a second stream for side=True, both routed GEMMs in FP8 for fp8=True; the
    Qwen3-shaped prefill's routed GEMMs run the persistent 256-row kernel):
    every replay, with eager work of the program between replays, gives the
    eager forward's bytes; new inputs written into the static tensors give
    the eager forward of those inputs (for bf16, matching the oracle)."""
    d = dev()
    cfg = SHARED_SMALL if name == "shared_small" else moe_synth.CONFIGS[name]
    say("graph", name, side, fp8)
    inp = inputs(cfg, d)
    kw = {}
    if fp8:
        kw = dict(w_down_fp8=mx.fp8_block_quant_weights(inp["w_down"]),
                  w_gate_up_fp8=mx.fp8_block_quant_weights(inp["w_gate_up"]))
    ref = _gpu_forward(cfg, inp, **kw).clone()
    stream = torch.cuda.Stream(d) if side else None
    g = mx.MoEForwardGraph(inp["hidden"].clone(), inp["logits"].clone(), inp["w_gate_up"], inp["w_down"], cfg.top_k,
                           cfg.rsf, cfg.padding_m, cfg.block_m, inp.get("shared_w_gate_up"), inp.get("shared_w_down"),
                           expert_bias=inp.get("bias"), scoring=cfg.scoring, renormalize=cfg.renormalize,
                           shared_stream=stream, **kw)
    for rep in range(3):
        g.out.zero_()
        other = _gpu_forward(cfg, inp, **kw)    # eager work between replays
        out = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        assert torch.equal(other, ref)
    # new inputs through the static tensors
    key = moe_synth.tensor_key(86, cfg.T)
    hid2 = moe_synth.normal_bf16(key, (cfg.T, cfg.H), 1.0, d)
    lg2 = moe_synth.normal_f32(key + 1, (cfg.T, cfg.E), 1.0, d)
    g.hidden.copy_(hid2)
    g.logits.copy_(lg2)
    out = g.replay().clone()
    inp2 = dict(inp, hidden=hid2, logits=lg2)
    ref2 = _gpu_forward(cfg, inp2, **kw)
    assert torch.equal(out, ref2)
    if name == "shared_small" and not fp8:
        exp = oracle_tokens(cfg, inp2, np.arange(cfg.T))
        assert_bf16_close(bits(out), exp["out"], "graph replay, new inputs")


@pytest.mark.parametrize("gate_up_fp8,side,shared_fp8", [(False, False, False), (False, True, False),
                                                         (True, False, False), (True, True, False),
                                                         (True, True, True)])
def test_forward_fp8(gate_up_fp8, side, shared_fp8):
    """The forward with its routed down projection in FP8 (h quantized to
    1x128-tile e4m3 codes, block-scaled FP8 grouped GEMM) and, with
    gate_up_fp8, its routed gate_up too (the hidden states quantized per
    token, read through the permutation): the same bytes as the stages called
    one by one (each checked against the oracle above), and within e4m3's
    quantization error of the oracle's bf16 forward: relative L2 error under
    5% with one FP8 GEMM, 8% with two or four (shared_fp8: the shared
    expert's GEMMs too; the codes' 3-bit mantissa sets about 2-3% per
    quantized operand; a wrong scale or a dropped block would be far above
    it)."""
    d = dev()
    cfg = SHARED_SMALL
    inp = inputs(cfg, d)
    qw = mx.fp8_block_quant_weights(inp["w_down"])
    qg = mx.fp8_block_quant_weights(inp["w_gate_up"]) if gate_up_fp8 else None
    qs = None
    if shared_fp8:
        qs = {"gate_up": mx.fp8_block_quant_weights(inp["shared_w_gate_up"]),
              "down": mx.fp8_block_quant_weights(inp["shared_w_down"])}
    stream = torch.cuda.Stream(d) if side else None
    out = _gpu_forward(cfg, inp, w_down_fp8=qw, w_gate_up_fp8=qg, w_shared_fp8=qs, shared_stream=stream).clone()
    # the same stages called one by one
    ids, w = mx.moe_topk_softmax(inp["logits"], cfg.top_k, scoring=cfg.scoring, renormalize=cfg.renormalize)
    tb = mx.moe_align(ids, cfg.E, cfg.padding_m, cfg.block_m)
    if gate_up_fp8:
        qh = mx.tile_quant_fp8(inp["hidden"], transposed=False)
        h = mx.grouped_gemm_gate_up_fp8(qh["q_row"], qh["s_row"], qg["q"], qg["s"], tb, cfg.padding_m,
                                        top_k=cfg.top_k)
    else:
        h = mx.grouped_gemm_gate_up_gather(inp["hidden"], inp["w_gate_up"], tb, cfg.top_k, cfg.padding_m,
                                           cfg.block_m)
    qa = mx.tile_quant_fp8(h, transposed=False)
    y = mx.grouped_gemm_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], tb, cfg.padding_m, cfg.block_m)
    if shared_fp8:
        qh = mx.tile_quant_fp8(inp["hidden"], transposed=False)
        shh = mx.grouped_gemm_gate_up_fp8(qh["q_row"], qh["s_row"], qs["gate_up"]["q"], qs["gate_up"]["s"], None, 128)
        qsh = mx.tile_quant_fp8(shh, transposed=False)
        sh = mx.grouped_gemm_fp8(qsh["q_row"], qsh["s_row"], qs["down"]["q"], qs["down"]["s"], None, 128)
    else:
        sh = mx.grouped_gemm_down(mx.grouped_gemm_gate_up(inp["hidden"], inp["shared_w_gate_up"], None, 128, 128),
                                  inp["shared_w_down"], None, 128, 128)
    ref = mx.moe_unpermute(y, tb["pair_to_row"], w, cfg.rsf, sh)
    assert torch.equal(out, ref)
    exp = oracle_tokens(cfg, inp, np.arange(cfg.T))["out"]
    o, e = nm.bf16_to_f64(bits(out)), nm.bf16_to_f64(exp)
    rel = np.linalg.norm(o - e) / np.linalg.norm(e)
    say("  fp8 forward relative L2 error vs the bf16 oracle", rel, "gate_up_fp8", gate_up_fp8)
    assert rel < (0.08 if gate_up_fp8 else 0.05), rel


def _full_batch_checks(cfg, inp, bufs, out, ref):
    """The whole batch against the oracle: each stage on the GPU's own input to
    that stage (bf16 results within atol = rtol = 1e-2 on every element, the
    SwiGLU byte for byte), then the output against the oracle's independent
    forward.

    With every token present, the oracle's compact rows (its experts are the
    reached ones, in ascending id) are the GPU's rows. End to end, the two
    sides round g and u, h and y to bf16 from differently ordered sums (fp32
    on the GPU, fp64 in the oracle), so a value within an accumulation error
    of a bf16 rounding boundary rounds to neighbouring bf16 values on the two
    sides, and a later stage scales the difference (the SwiGLU by silu(g) or
    u, the unpermute by rsf * w, rsf up to 2.827 here). So an output element
    may leave atol + rtol*|ref| only by what the unpermute's linearity gives
    for the y and weight differences, rsf * sum_j (w_j |dy_j| + |dw_j| |y_j|)
    plus the shared output's difference, plus one ulp of the output for its
    rounding; the y differences themselves are bounded by the stage checks.
    """
    h_gpu, y_gpu = bits(bufs.h), bits(bufs.y)
    assert h_gpu.shape == ref["h"].shape and y_gpu.shape == ref["y"].shape
    tab = ref["tables"]
    d = bufs.h.device
    # stage: the gate_up GEMM (unfused, gathering the hidden states) against the oracle's
    gu = mx.grouped_gemm_gate_up_gather(inp["hidden"], inp["w_gate_up"], bufs.tables, cfg.top_k, cfg.padding_m,
                                        cfg.block_m, False)
    gu_gpu = bits(gu)
    del gu
    err = assert_bf16_close(gu_gpu, ref["gate_up"], f"{cfg.name} gate_up")
    say("  gate_up max abs err", err)
    # stage: the SwiGLU fused into the forward's gate_up, byte for byte on the GPU's g|u
    h_spec = oracle.swiglu(gu_gpu, cfg.F)
    assert np.array_equal(h_gpu, h_spec), f"{cfg.name}: {int((h_gpu != h_spec).sum())} h values differ"
    del gu_gpu, h_spec
    # stage: down projection of the GPU's h
    y_from_h = oracle.grouped_gemm(h_gpu, ref["w_down_used"], tab["group_sizes"], tab["group_offsets"])
    err = assert_bf16_close(y_gpu, y_from_h, f"{cfg.name} y from the GPU's h")
    say("  y (from the GPU's h) max abs err", err)
    del y_from_h
    # stage: unpermute of the GPU's y (and shared output)
    shared_gpu = bits(bufs.shared_y) if cfg.shared_F else None
    w = host(bufs.topk_weights)
    out_from_y = oracle.unpermute(y_gpu, tab["pair_to_row"], w, cfg.top_k, cfg.rsf, shared_gpu)
    out_gpu = bits(out)
    err = assert_bf16_close(out_gpu, out_from_y, f"{cfg.name} out from the GPU's y")
    say("  out (from the GPU's y) max abs err", err)
    # end to end, against the oracle's own forward
    _assert_within_propagated(cfg, out_gpu, ref["out"], y_gpu, ref, w, tab, shared_gpu, "out")


def _assert_within_propagated(cfg, got_bits, ref_bits, y_gpu, ref, w, tab, shared_gpu, what):
    """got against the oracle's forward output: within atol + rtol*|ref| on all
    but at most 1e-5 of the elements, and every element within that plus the
    unpermute's propagation of the y and weight differences (plus the shared
    output's difference when it joined) plus one output ulp."""
    g, r = nm.bf16_to_f64(got_bits), nm.bf16_to_f64(ref_bits)
    diff = np.abs(g - r)
    tol = BF16_ATOL + BF16_RTOL * np.abs(r)
    outside = diff > tol
    rows = np.asarray(tab["pair_to_row"], np.int64).reshape(cfg.T, cfg.top_k)
    prop = np.zeros_like(g)
    rsf = float(np.float32(cfg.rsf))
    dw = np.abs(w.astype(np.float64) - ref["topk_weights"].astype(np.float64))
    for j in range(cfg.top_k):
        yg = nm.bf16_to_f64(y_gpu[rows[:, j]])
        dy = np.abs(yg - nm.bf16_to_f64(ref["y"][rows[:, j]]))
        prop += rsf * (w[:, j:j + 1].astype(np.float64) * dy + dw[:, j:j + 1] * np.abs(yg))
    if shared_gpu is not None:
        prop += np.abs(nm.bf16_to_f64(shared_gpu) - nm.bf16_to_f64(ref["shared"]))
    bound = tol + prop + bf16_ulp(ref_bits)
    bad = diff > bound
    say(f"  {what} vs the oracle's forward: max abs err", float(diff.max()), "outside atol/rtol:",
        int(outside.sum()), "of", diff.size, "(all within the propagated bound)" if not bad.any() else "")
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the propagated bound; first "
                           f"{np.argwhere(bad)[:5].tolist()}")
    assert outside.sum() <= 1e-5 * diff.size, int(outside.sum())


# sampled tokens per workload: each one brings up to k experts' weights to the
# host; None: every token (the whole batch against the oracle's forward)
SAMPLED_TOKENS = {"qwen3_prefill": None, "dsv3_prefill": None, "kimi_k2_t32": 3, "kimi_k2_t512": 3,
                  "kimi_k2_t2048": 3, "kimi_k2_t4096": 3}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["qwen3_prefill", "dsv3_prefill", "kimi_k2_t32", "kimi_k2_t512", "kimi_k2_t2048",
                                  "kimi_k2_t4096"])
def test_forward_full_size_sampled_tokens(name):
    d = dev()
    cfg = moe_synth.CONFIGS[name]
    say("forward", name, "generating inputs")
    inp = inputs(cfg, d)
    bufs = mx.MoEBuffers(mx.MoEShape(cfg.T, cfg.H, cfg.F, cfg.E, cfg.top_k, cfg.padding_m, cfg.block_m,
                                     cfg.shared_F), d)
    out = _gpu_forward(cfg, inp, buffers=bufs)
    torch.cuda.synchronize()
    # full-size tables against the oracle's
    ids = host(bufs.topk_ids)
    ref_ids, _ = oracle.route(host(inp["logits"]), cfg.top_k, host(inp["bias"]) if "bias" in inp else None,
                              cfg.scoring, cfg.renormalize)
    assert np.array_equal(ids, ref_ids)
    ref_tab = oracle.dispatch_tables(ref_ids, cfg.E, cfg.padding_m, cfg.block_m)
    for key in ("group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx", "sorted_pair",
                "pair_to_row"):
        assert np.array_equal(host(bufs.tables[key]), ref_tab[key]), key
    say("  active experts", int((ref_tab["group_sizes"] > 0).sum()), "max rows", int(ref_tab["group_sizes"].max()))
    if SAMPLED_TOKENS[name] is None:
        tokens = np.arange(cfg.T)
    else:
        tokens = np.unique(np.concatenate([[0, 1, cfg.T - 1],
                                           np.random.default_rng(cfg.cid).choice(cfg.T, SAMPLED_TOKENS[name])]))
    say("  oracle on", tokens.size, "tokens")
    ref = oracle_tokens(cfg, inp, tokens)
    if SAMPLED_TOKENS[name] is None:
        _full_batch_checks(cfg, inp, bufs, out, ref)
    else:
        err = assert_bf16_close(bits(out[torch.as_tensor(tokens, device=d)]), ref["out"], f"{name} out")
        say("  out max abs err over", tokens.size, "tokens", err)
    if cfg.shared_F:
        assert_bf16_close(bits(bufs.shared_y[torch.as_tensor(tokens, device=d)]), ref["shared"], "shared")
    # determinism: a second forward gives the same bytes
    out2 = _gpu_forward(cfg, inp)
    assert torch.equal(out, out2)
    if cfg.shared_F:
        # the shared expert on a second stream, concurrent with the routed path: same bytes
        ref_out, ref_shared = out.clone(), bufs.shared_y.clone()
        side = torch.cuda.Stream(d)
        for _ in range(2):
            bufs.out.zero_()
            bufs.shared_y.zero_()
            out3 = _gpu_forward(cfg, inp, buffers=bufs, shared_stream=side)
            assert torch.equal(out3, ref_out) and torch.equal(bufs.shared_y, ref_shared)
        shared_o, routed_o = _gpu_forward(cfg, inp, buffers=bufs, return_parts=True, shared_stream=side)
        assert torch.equal(shared_o, ref_shared)
        # the split of the partial-output contract: shared part and routed part, added by the caller
        shared, routed = _gpu_forward(cfg, inp, return_parts=True)
        assert torch.equal(shared, bufs.shared_y)
        if SAMPLED_TOKENS[name] is None:
            _assert_within_propagated(cfg, bits(routed), ref["routed"], bits(bufs.y), ref, host(bufs.topk_weights),
                                      ref["tables"], None, "routed part")
        else:
            sel = torch.as_tensor(tokens, device=d)
            assert_bf16_close(bits(routed[sel]), ref["routed"], f"{name} routed part")
