"""Host-side checks of the seeded workload definitions (no GPU)."""
import numpy as np

import moe_synth


def test_aligned_gemm_cases_follow_the_table():
    """E = T // M for the token counts of the TileOPs grouped-GEMM baseline table
    (PR #1580, "Benchmark results - grouped-GEMM baselines"); N and K as printed."""
    table_T = {"glm5_up_t32768": 32768, "glm5_up_t65536": 65536, "glm5_up_t131072": 131072,
               "glm5_up_t262144": 262144, "glm5_down_t32768": 32768, "glm5_down_t65536": 65536,
               "glm5_down_t131072": 131072, "glm5_down_t262144": 262144,
               "llama4_128e_up_t131072": 131072, "llama4_128e_down_t131072": 131072,
               "qwen3.5_397b_up_t52429": 52429, "qwen3.5_397b_down_t52429": 52429}
    assert set(table_T) == set(moe_synth.GEMM_CASES)
    for name, T in table_T.items():
        c = moe_synth.GEMM_CASES[name]
        assert c.E == T // c.M, name
        assert c.N % 256 == 0 and c.K % 64 == 0, name
    assert len({c.cid for c in moe_synth.GEMM_CASES.values()}) == len(table_T)


def test_aligned_gemm_inputs_are_keyed_per_expert():
    """A weight slice regenerated for one expert equals that expert's slice of the whole tensor."""
    c = moe_synth.GemmCase(99, "probe", M=4, N=8, K=16, E=3, page_tflops=0.0)
    w = moe_synth.gemm_w(c)
    for e in range(3):
        assert np.array_equal(moe_synth.bits16(moe_synth.gemm_w(c, experts=[e])[0]), moe_synth.bits16(w[e]))
    a = moe_synth.gemm_a(c)
    assert np.array_equal(moe_synth.bits16(moe_synth.gemm_a(c, rows=slice(5, 9))), moe_synth.bits16(a[5:9]))


def test_router_logits_are_normal_with_tails():
    """The router logits are drawn from a true N(0, 1): mean, variance and the
    mass beyond 3 sigma (2.70e-3 for a normal; a four-uniform sum gives about
    2e-4) on the 4096 x 256 logits of the DeepSeek-V3-shaped workload."""
    cfg = moe_synth.CONFIGS["dsv3_prefill"]
    z = moe_synth.router_logits(cfg).numpy().astype(np.float64)
    assert z.dtype == np.float64 and z.shape == (cfg.T, cfg.E)
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    tail = (np.abs(z) > 3.0).mean()
    # binomial sd of the tail fraction at p = 2.70e-3 over 2^20 draws: 5.1e-5
    assert abs(tail - 2.6998e-3) < 5 * 5.1e-5, tail
    assert np.abs(z).max() > 4.5


def test_router_logits_rows_are_prefixes():
    """A row range is a slice of the stream, and a smaller token count of one
    workload id takes the first rows of the larger one's logits."""
    big = moe_synth.CONFIGS["kimi_k2_t4096"]
    small = moe_synth.CONFIGS["kimi_k2_t32"]
    z = moe_synth.router_logits(big).numpy()
    assert np.array_equal(moe_synth.router_logits(small).numpy(), z[:32])
    assert np.array_equal(moe_synth.router_logits(big, rows=slice(7, 11)).numpy(), z[7:11])


def test_dsv3_skewed_routing_reach():
    """N(0, 1) logits plus the Zipf(1.1) rank bias reach about 160-170 of the
    256 experts with the largest group near 3970 rows (the config's skew: some
    experts get no tokens, the others unaligned counts)."""
    import oracle
    cfg = moe_synth.CONFIGS["dsv3_prefill"]
    ids, _ = oracle.route(moe_synth.router_logits(cfg).numpy(), cfg.top_k, moe_synth.zipf_bias(cfg))
    gs = np.bincount(ids.ravel(), minlength=cfg.E)
    active = int((gs > 0).sum())
    assert 155 <= active <= 172, active
    assert 3900 <= gs.max() <= 4050, gs.max()
    assert (gs[gs > 0] % 128 != 0).sum() >= active - 3
