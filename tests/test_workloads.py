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
