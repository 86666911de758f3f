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


# ------------------------------------------------ grouped (expand_128x) --

PAGE_GROUPS = [0, 1, 127, 128, 129]     # the grouped quantizers' test sizes in xtuner #2089


def _grouped_h(sizes, K, key=81):
    M = int(sum(sizes))
    return moe_synth.bits16(moe_synth.normal_bf16(moe_synth.tensor_key(key, M, K), (M, K), 1.0))


def test_expand_128x_offsets_of_the_page_sizes():
    """[0, 1, 127, 128, 129] rows expand to [0, 128, 128, 128, 256] columns:
    groups start at columns 0, 0, 128, 256, 384 of a 640-column q_t."""
    starts, total = oracle.expand_128x_starts(PAGE_GROUPS)
    assert starts == [0, 0, 128, 256, 384] and total == 640
    h = _grouped_h(PAGE_GROUPS, 256)
    for trans, s_rows in (("block", 2), ("tile", 256)):
        q = oracle.quant_fp8_grouped(h, PAGE_GROUPS, trans)
        assert q["q_t"].shape == (256, 640) and q["s_t"].shape == (s_rows, 5)
        assert q["q_row"].shape == (385, 256) and q["s_row"].shape == (385, 2)
        # pad columns of each group are zero: group 1 uses 1 of 128, group 2 127, group 4 129 of 256
        assert not q["q_t"][:, 1:128].any() and not q["q_t"][:, 255:256].any()
        assert not q["q_t"][:, 384 + 129:].any()


def test_grouped_block_mode_with_one_group_is_the_plain_quantizer():
    for M in (1, 127, 300):
        h = _grouped_h([M], 256, key=82)
        a, b = oracle.quant_fp8_grouped(h, None, "block"), oracle.quant_fp8(h)
        for k in ("q_row", "s_row", "q_t", "s_t"):
            assert np.array_equal(a[k], b[k]), (M, k)


@pytest.mark.parametrize("sizes", [PAGE_GROUPS, [300, 0, 0, 5, 256]])
def test_grouped_layout_is_each_group_quantized_alone(sizes):
    """Group g's columns of q_t (and s_t) are what the plain quantizer gives
    for g's rows alone, at the group's expanded offset; the row layout is the
    plain one of all rows."""
    K = 256
    h = _grouped_h(sizes, K, key=83)
    q = oracle.quant_fp8_grouped(h, sizes, "block", m_pad=1024)
    whole = oracle.quant_fp8(h)
    assert np.array_equal(q["q_row"], whole["q_row"]) and np.array_equal(q["s_row"], whole["s_row"])
    starts, total = oracle.expand_128x_starts(sizes)
    r0 = 0
    for n, c0 in zip(sizes, starts):
        if n:
            alone = oracle.quant_fp8(h[r0:r0 + n])
            w = alone["q_t"].shape[1]
            assert np.array_equal(q["q_t"][:, c0:c0 + w], alone["q_t"])
            assert np.array_equal(q["s_t"][:, c0 // 128:(c0 + w) // 128], alone["s_t"])
        r0 += n
    assert not q["q_t"][:, total:].any() and not q["s_t"][:, total // 128:].any()


@pytest.mark.parametrize("sizes", [PAGE_GROUPS, [1, 300]])
def test_grouped_tile_mode_is_the_row_quantizer_on_each_transposed_group(sizes):
    """Per-tile transposed scales run along the rows of one column, 128 rows of
    a group at a time: that is the row-layout (1x128) quantizer applied to the
    group's transpose, zero-padded to its expanded width (zeros change no
    amax and encode as 0x00)."""
    K = 256
    h = _grouped_h(sizes, K, key=84)
    q = oracle.quant_fp8_grouped(h, sizes, "tile")
    starts, _ = oracle.expand_128x_starts(sizes)
    r0 = 0
    for n, c0 in zip(sizes, starts):
        if n:
            w = -(-n // 128) * 128
            ht = np.zeros((K, w), np.uint16)
            ht[:, :n] = h[r0:r0 + n].T
            rq = oracle.quant_fp8(ht)
            assert np.array_equal(q["q_t"][:, c0:c0 + w], rq["q_row"])
            assert np.array_equal(q["s_t"][:, c0 // 128:(c0 + w) // 128], rq["s_row"])
        r0 += n


def test_grouped_tile_mode_brute_force():
    """Per-element check of a few tiles: scale = fl32(amax/448) over the
    tile's real rows of one column, code = e4m3(fl32(h/s))."""
    sizes = [5, 140]
    h = _grouped_h(sizes, 128, key=85)
    hf = nm.bf16_to_f32(h)
    q = oracle.quant_fp8_grouped(h, sizes, "tile")
    # group 1, second tile: rows 5 + 128 .. 5 + 139 -> columns 128 + 128 .. 128 + 139
    for col in (0, 63, 127):
        rows = range(133, 145)
        amax = max(abs(float(hf[m, col])) for m in rows)
        s = np.float32(np.float32(amax) / np.float32(448.0))
        assert q["s_t"][col, 2] == s
        for m in rows:
            code = nm.e4m3_encode(np.array([np.float32(hf[m, col]) / s], np.float32))[0]
            assert q["q_t"][col, 256 + (m - 133)] == code
    assert not q["q_t"][:, 5:128].any() and not q["q_t"][:, 268:].any()


def test_grouped_rejects_bad_sizes():
    h = _grouped_h([4], 128, key=86)
    with pytest.raises(ValueError):
        oracle.quant_fp8_grouped(h, [3], "block")
    with pytest.raises(ValueError):
        oracle.quant_fp8_grouped(h, [4], "block", m_pad=64)
    with pytest.raises(ValueError):
        oracle.quant_fp8_grouped(h, [4], "row")


# ------------------------------------------ block-scaled FP8 GEMM (oracle) --

def test_block_weight_quant_is_the_transposed_activation_layout():
    """A 128x128 block of the weight is quantized as a block of the transposed
    activation layout: block_quant_fp8(W) == quant_fp8(W^T)'s (q_t, s_t)."""
    w = moe_synth.bits16(moe_synth.normal_bf16(moe_synth.tensor_key(87), (256, 384), 0.05))
    b = oracle.block_quant_fp8(w)
    t = oracle.quant_fp8(np.ascontiguousarray(w.T))
    assert np.array_equal(b["q"], t["q_t"]) and np.array_equal(b["s"], t["s_t"])
    # every non-zero block holds a code of magnitude 448
    for nb in range(2):
        for kb in range(3):
            blk = b["q"][nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert ((blk & 0x7F) == 0x7E).any()


def test_fp8_gemm_exact_on_integer_codes():
    """Codes that decode to small integers with unit scales (and power-of-two
    scales, which commute with every rounding): the result is the exact integer
    product, so a transposed operand, a wrong scale index or a dropped block
    shows up. Three groups, one empty, one ragged."""
    rng = np.random.default_rng(5)
    sizes = np.array([3, 0, 130], np.int64)
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    M, N, K = int(sizes.sum()), 128, 256
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0])     # 0, 1, 2, 3, 4, -1, -2
    vals = nm.e4m3_decode(ints)
    ia = rng.integers(0, len(ints), (M, K))
    iw = rng.integers(0, len(ints), (3, N, K))
    qa, qw = ints[ia].astype(np.uint8), ints[iw].astype(np.uint8)
    for sa_v, sw_v in ((1.0, 1.0), (0.5, 4.0)):
        sa = np.full((M, K // 128), sa_v, np.float32)
        sw = np.full((3, N // 128, K // 128), sw_v, np.float32)
        y = oracle.grouped_gemm_fp8(qa, sa, qw, sw, sizes, offs)
        for e in (0, 2):
            o, n = int(offs[e]), int(sizes[e])
            exact = (vals[ia[o:o + n]] @ vals[iw[e]].T) * sa_v * sw_v
            assert np.array_equal(nm.bf16_to_f64(y[o:o + n]), nm.bf16_to_f64(nm.to_bf16(exact)))


def test_fp8_gemm_scales_apply_per_block():
    """Brute force on one output: sum over 128-column blocks of
    (decoded a * a-scale of the row's block) * (decoded w * w-scale of its block)."""
    rng = np.random.default_rng(6)
    M, N, K = 4, 256, 384
    qa = rng.integers(0, 0x7E, (M, K)).astype(np.uint8)
    qw = rng.integers(0, 0x7E, (1, N, K)).astype(np.uint8)
    sa = rng.uniform(0.01, 2.0, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.01, 2.0, (1, N // 128, K // 128)).astype(np.float32)
    y = oracle.grouped_gemm_fp8(qa, sa, qw, sw, np.array([M]), np.array([0]))
    for m, n in ((0, 0), (3, 255), (2, 129)):
        acc = 0.0
        for k in range(K):
            acc += (nm.e4m3_decode(qa[m, k:k + 1])[0] * float(sa[m, k // 128])) * \
                   (nm.e4m3_decode(qw[0, n, k:k + 1])[0] * float(sw[0, n // 128, k // 128]))
        assert nm.bf16_to_f64(y[m:m + 1, n])[0] == nm.bf16_to_f64(nm.to_bf16(np.array([acc])))[0]
