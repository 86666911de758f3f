"""Pins for the oracle's SwiGLU + FP8 quantizer.

A hand-worked tile (amax 448 makes the scale exactly 1, so the codes are the
plain e4m3 encodings of the values), a per-element brute force of the
transposed layout, and the invariants any correct 1x128 / 128x128 absmax
quantizer has: the tile maximum maps to code 448, dequantisation error is at
most half a code step, zero tiles give zero, pad columns stay zero.
"""
import numpy as np
import pytest

import moe_synth
import oracle
from oracle import numerics as nm


def test_hand_worked_tile():
    vals = np.zeros((1, 128))
    vals[0, :8] = [448.0, 1.0, -0.5, 3.0, 0.0, 2.0 ** -9, -448.0, 0.001953125 * 0.75]
    h = nm.to_bf16(vals)
    q = oracle.quant_fp8(h)
    assert q["s_row"].tolist() == [[1.0]]
    assert q["q_row"][0, :8].tolist() == [0x7E, 0x38, 0xB0, 0x44, 0x00, 0x01, 0xFE, 0x01]
    assert q["s_t"].tolist() == [[1.0]]
    assert q["q_t"].shape == (128, 128)
    assert q["q_t"][:8, 0].tolist() == q["q_row"][0, :8].tolist()
    assert not q["q_t"][:, 1:].any()                          # pad columns of rows 1..127


def test_zero_tiles_and_edge_sizes():
    for M in moe_synth.QUANT_EDGE_M:
        x = moe_synth.bits16(moe_synth.quant_input(M, 256))
        q = oracle.swiglu_quant_fp8(x, 256)
        mp = -(-M // 128) * 128
        assert q["q_row"].shape == (M, 256) and q["s_row"].shape == (M, 2)
        assert q["q_t"].shape == (256, mp) and q["s_t"].shape == (2, mp // 128)
        if M:
            assert not q["q_t"][:, M:].any()
    h = np.zeros((3, 128), np.uint16)
    h[1, 5] = 0x8000                                           # -0.0 alone is still a zero tile
    q = oracle.quant_fp8(h)
    assert not q["q_row"].any() and not q["s_row"].any() and not q["s_t"].any()


@pytest.mark.parametrize("M", [1, 129, 300])
def test_transposed_layout_brute_force(M):
    F = 256
    x = moe_synth.bits16(moe_synth.quant_input(M, F))
    q = oracle.swiglu_quant_fp8(x, F)
    h = nm.bf16_to_f32(q["h"])
    for fb in range(F // 128):
        for mb in range(-(-M // 128)):
            rows = range(mb * 128, min(M, mb * 128 + 128))
            amax = max(abs(float(h[m, f])) for m in rows for f in range(fb * 128, fb * 128 + 128))
            s = np.float32(np.float32(amax) / np.float32(448.0))
            assert q["s_t"][fb, mb] == s
            for m in list(rows)[:3] + list(rows)[-2:]:
                for f in (fb * 128, fb * 128 + 77, fb * 128 + 127):
                    code = nm.e4m3_encode(np.array([np.float32(h[m, f]) / s], np.float32))[0]
                    assert q["q_t"][f, m] == code


def test_quant_invariants_on_workload_rows():
    F = 2048
    x = moe_synth.bits16(moe_synth.quant_input(1024, F, rows=slice(0, 160)))
    q = oracle.swiglu_quant_fp8(x, F)
    h = nm.bf16_to_f64(q["h"])
    s = q["s_row"].astype(np.float64)
    # the largest magnitude of every non-zero tile maps to 448 (code 0x7E / 0xFE)
    codes = q["q_row"].reshape(160, F // 128, 128)
    assert np.all((codes & 0x7F).max(axis=2)[s > 0] == 0x7E)
    # dequantisation error at most half the e4m3 spacing at that value (times s)
    deq = nm.e4m3_decode(q["q_row"]).reshape(160, F // 128, 128) * s[:, :, None]
    v = h.reshape(160, F // 128, 128)
    a = np.abs(v / s[:, :, None])
    step = np.where(a >= 2 ** -6, np.ldexp(1.0, np.frexp(a)[1] - 1 - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - v) <= 0.5 * step * s[:, :, None] * (1 + 1e-6) + 1e-45)
    # the transposed block scale is the max of its rows' tile scales (same amax)
    sb = q["s_t"][:, 0]
    np.testing.assert_array_equal(sb, q["s_row"][:128].max(axis=0))
    # swiglu_quant_fp8 equals quantizing the separately computed SwiGLU
    q2 = oracle.quant_fp8(oracle.swiglu(x, F))
    for key in ("q_row", "s_row", "q_t", "s_t"):
        assert np.array_equal(q[key], q2[key])
