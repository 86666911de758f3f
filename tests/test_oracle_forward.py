"""Pins for the oracle's GEMM, SwiGLU, unpermute and whole forward.

* grouped_gemm: a pure-Python exactly rounded dot product (math.fsum) on tiny
  inputs, and a closed form with one-hot weight rows that fixes which operand
  is transposed and which expert's weights a row meets.
* swiglu: closed forms (up = 1 gives SiLU(gate) alone; gate|up order).
* forward: a per-token computation that never builds the dispatch tables or
  the permutation, against the grouped pipeline.
* unpermute: exact linearity in routed_scaling_factor for powers of two,
  one-rounding bound for rsf = 2.827.
"""
import math
import random

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from oracle import numerics as nm


def _rand_bf16(rng, shape, scale=1.0):
    return nm.to_bf16(rng.standard_normal(shape) * scale)


def test_grouped_gemm_fsum_brute_force():
    rng = np.random.default_rng(11)
    E, N, K = 3, 5, 37
    sizes = np.array([4, 0, 3], dtype=np.int32)
    offs = np.array([0, 4, 4], dtype=np.int32)
    a = _rand_bf16(rng, (7, K))
    w = _rand_bf16(rng, (E, N, K), 0.3)
    out = oracle.grouped_gemm(a, w, sizes, offs)
    af, wf = nm.bf16_to_f64(a), nm.bf16_to_f64(w)
    for e in range(E):
        for r in range(offs[e], offs[e] + sizes[e]):
            for n in range(N):
                exact = math.fsum(float(af[r, kk]) * float(wf[e, n, kk]) for kk in range(K))
                assert out[r, n] == nm.to_bf16(np.array([exact]))[0]


def test_grouped_gemm_one_hot_weights_pick_columns():
    # W[e][n] = unit vector at column c(e, n): C[r, n] = A[r, c(e, n)] exactly
    rng = np.random.default_rng(12)
    E, N, K = 3, 6, 9
    a = _rand_bf16(rng, (10, K))
    pick = rng.integers(0, K, size=(E, N))
    w = np.zeros((E, N, K), dtype=np.uint16)
    for e in range(E):
        for n in range(N):
            w[e, n, pick[e, n]] = 0x3F80                    # bf16 1.0
    sizes = np.array([2, 5, 3], np.int32)
    offs = np.array([0, 2, 7], np.int32)
    out = oracle.grouped_gemm(a, w, sizes, offs)
    for e in range(E):
        for r in range(offs[e], offs[e] + sizes[e]):
            assert out[r].tolist() == a[r, pick[e]].tolist()


def test_swiglu_closed_forms():
    rng = np.random.default_rng(5)
    M, F = 4, 8
    g = _rand_bf16(rng, (M, F), 2.0)
    one = np.full((M, F), 0x3F80, np.uint16)
    h = oracle.swiglu(np.concatenate([g, one], axis=1), F)
    assert np.array_equal(h, nm.to_bf16(nm.silu32(nm.bf16_to_f32(g))))
    # swapping the halves gives SiLU(1) * g, not SiLU(g)
    h2 = oracle.swiglu(np.concatenate([one, g], axis=1), F)
    s1 = nm.silu32(np.array([1.0], np.float32))[0]
    assert np.array_equal(h2, nm.to_bf16((s1 * nm.bf16_to_f32(g)).astype(np.float32)))
    # silu(g) * up against float64 math within bf16 rounding
    u = _rand_bf16(rng, (M, F))
    h3 = nm.bf16_to_f64(oracle.swiglu(np.concatenate([g, u], axis=1), F))
    gf, uf = nm.bf16_to_f64(g), nm.bf16_to_f64(u)
    np.testing.assert_allclose(h3, gf / (1 + np.exp(-gf)) * uf, rtol=2 ** -8, atol=1e-30)


def _per_token_forward(hid, logits, wgu, wd, k, rsf, shared=None, bias=None):
    """Token by token: no tables, no permutation, same rounding points."""
    ids, w = oracle.route(logits, k, bias)
    T, H = hid.shape
    F = wd.shape[2]
    out = np.zeros((T, H), np.uint16)
    x = nm.bf16_to_f64(hid)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = int(ids[t, j])
            gu = nm.to_bf16(nm.bf16_to_f64(wgu[e]) @ x[t])
            g, u = nm.bf16_to_f32(gu[:F]), nm.bf16_to_f32(gu[F:])
            h = nm.to_bf16((nm.silu32(g) * u).astype(np.float32))
            y = nm.to_bf16(nm.bf16_to_f64(wd[e]) @ nm.bf16_to_f64(h))
            acc += float(w[t, j]) * nm.bf16_to_f64(y)
        val = float(np.float32(rsf)) * acc
        if shared is not None:
            val = val + nm.bf16_to_f64(shared[t])
        out[t] = nm.to_bf16(val)
    return out


def _tiny_inputs(cfg):
    return (moe_synth.bits16(moe_synth.hidden(cfg)), moe_synth.router_logits(cfg).numpy(),
            moe_synth.bits16(moe_synth.w_gate_up(cfg)), moe_synth.bits16(moe_synth.w_down(cfg)))


def test_forward_matches_per_token_computation():
    cfg = moe_synth.CONFIGS["tiny"]
    hid, logits, wgu, wd = _tiny_inputs(cfg)
    res = oracle.forward(hid, logits, wgu, wd, cfg.top_k, cfg.rsf, cfg.padding_m, cfg.block_m)
    ref = _per_token_forward(hid, logits, wgu, wd, cfg.top_k, cfg.rsf)
    assert np.array_equal(res["out"], ref)
    # the fused reading: gate_up rounded to bf16, then SwiGLU
    assert np.array_equal(res["h"], oracle.swiglu(res["gate_up"], cfg.F))


def test_forward_with_shared_expert_and_skew():
    cfg = moe_synth.MoEConfig(90, "tiny_shared", T=24, H=64, F=128, E=16, top_k=4, padding_m=32,
                              block_m=16, rsf=2.827, zipf_s=1.1, shared_F=128)
    hid, logits, wgu, wd = _tiny_inputs(cfg)
    bias = moe_synth.expert_bias(cfg).numpy()
    swgu = moe_synth.bits16(moe_synth.shared_w_gate_up(cfg))
    swd = moe_synth.bits16(moe_synth.shared_w_down(cfg))
    res = oracle.forward(hid, logits, wgu, wd, cfg.top_k, cfg.rsf, cfg.padding_m, cfg.block_m,
                         swgu, swd, bias=bias)
    # shared expert per token, by the same no-table route
    x = nm.bf16_to_f64(hid)
    shared = np.zeros_like(hid)
    for t in range(cfg.T):
        gu = nm.to_bf16(nm.bf16_to_f64(swgu) @ x[t])
        h = nm.to_bf16((nm.silu32(nm.bf16_to_f32(gu[:cfg.shared_F])) *
                        nm.bf16_to_f32(gu[cfg.shared_F:])).astype(np.float32))
        shared[t] = nm.to_bf16(nm.bf16_to_f64(swd) @ nm.bf16_to_f64(h))
    assert np.array_equal(res["shared"], shared)
    ref = _per_token_forward(hid, logits, wgu, wd, cfg.top_k, cfg.rsf, shared, bias)
    assert np.array_equal(res["out"], ref)
    assert (res["group_sizes"] == 0).any()          # the skew leaves some experts empty


def test_unpermute_linearity_in_scaling_factor():
    cfg = moe_synth.CONFIGS["tiny"]
    hid, logits, wgu, wd = _tiny_inputs(cfg)
    res = oracle.forward(hid, logits, wgu, wd, cfg.top_k, 1.0, cfg.padding_m, cfg.block_m)
    y, p2r, w = res["y"], res["pair_to_row"], res["topk_weights"]
    o1 = nm.bf16_to_f64(oracle.unpermute(y, p2r, w, cfg.top_k, 1.0))
    for rsf in (2.0, 0.5, 4.0):
        o = nm.bf16_to_f64(oracle.unpermute(y, p2r, w, cfg.top_k, rsf))
        assert np.array_equal(o, rsf * o1)                      # power-of-two scaling is exact
    rsf = 2.827
    o = nm.bf16_to_f64(oracle.unpermute(y, p2r, w, cfg.top_k, rsf))
    r32 = float(np.float32(rsf))
    ulp = lambda v: np.ldexp(1.0, np.frexp(np.abs(v))[1] - 8)  # noqa: E731  bf16 spacing
    assert np.all(np.abs(o - r32 * o1) <= 0.5 * ulp(o) + r32 * 0.5 * ulp(o1) + 1e-30)
    assert np.abs(o).max() > 0


def test_unpermute_weights_and_rows():
    # one-hot y rows: out[t] picks w[t,j] at the row each slot maps to
    T, k, H = 3, 2, 4
    y = np.zeros((T * k, H), np.uint16)
    for r in range(T * k):
        y[r, r % H] = 0x3F80
    p2r = np.array([5, 0, 1, 4, 2, 3], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [1.0, 0.0]], np.float32)
    out = nm.bf16_to_f64(oracle.unpermute(y, p2r, w, k, 1.0))
    exp = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            exp[t, p2r[t * k + j] % H] += w[t, j]
    assert np.array_equal(out, exp)


def test_synth_generator_is_device_independent_and_sliceable():
    cfg = moe_synth.CONFIGS["tiny"]
    w = moe_synth.w_down(cfg)
    assert torch.equal(moe_synth.w_down(cfg, experts=[6, 1]), w[[6, 1]])
    x = moe_synth.normal_f32(moe_synth.tensor_key(1, 2), (1 << 16,))
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    assert float(x.abs().max()) < 3.5
