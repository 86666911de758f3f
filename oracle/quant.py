"""Oracle for the fused SwiGLU + 1x128-tile FP8 (e4m3) activation quantizer.

Test infrastructure only (see oracle/__init__.py).

xtuner #2089 ("Summary", "Changes") describes the kernels this restates:
  * per_tile_quant: row layout, one scale per 1x128 tile of a row;
  * trans_per_block_quant_expand_128x: the transposed layout with one scale
    per 128x128 block, the row count expanded to a multiple of 128;
  * swiglu_per_tile_quant_with_trans_per_block: SiLU(gate) * up followed by
    both layouts in one pass, equal byte for byte to running the SwiGLU and
    the two quantizers one after the other ("Correctness"; the review thread
    asks for bitwise comparisons).
  * per_tile_quant_with_trans_per_block / per_tile_quant_with_trans_per_tile:
    the same two layouts without the SwiGLU, on an activation whose rows are
    grouped by expert; the transposed copy is "expand_128x" per group (its
    tests use group sizes such as [0, 1, 127, 128, 129] with 6144 columns),
    and its scales are per 128x128 block or per 128-row tile of one column.
The workload fixes the format (OCP e4m3, max 448) and the fp32 scale
amax / 448.

Readings where the pages are silent (each side implements the same):
  * s = fl32(amax / 448) and code = e4m3(fl32(h / s)) with correctly rounded
    fp32 divisions; a tile whose amax is 0 gets s = 0 and all codes 0x00.
  * Layouts: q_row [M, F] uint8, s_row [M, F/128] float32 (row-major);
    q_t [F, M_pad] uint8 with M_pad = ceil(M/128)*128 and zero bytes in the
    pad columns; s_t [F/128, M_pad/128] float32 (row-major). The transposed
    block's amax runs over real rows only.
  * The SwiGLU value quantized is the bf16 one (see moe.swiglu), which is what
    makes the fused kernel equal to the unfused pair.
  * Grouped ("expand_128x") transposed layout: the groups are consecutive row
    ranges of the given sizes; group g's rows fill ceil(s_g/128)*128 columns of
    q_t starting at the sum of the previous groups' padded sizes (an empty
    group takes none), pad columns hold 0x00, and a 128-row tile never spans
    two groups. Per-block scales: s_t [K/128, m_pad/128]; per-tile scales (one
    per column and 128-row tile of a group, amax over its real rows): s_t
    [K, m_pad/128]. Columns past the groups' padded total (when the caller's
    width m_pad is larger) hold 0x00 and their scales 0.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .moe import swiglu
from .numerics import E4M3_MAX, bf16_to_f32, bf16_to_f64, e4m3_decode, e4m3_encode, to_bf16

TILE = 128
F32 = np.float32


def _tile_codes(vals: np.ndarray, amax: np.ndarray):
    """Scale and codes for values whose tile amax broadcasts against them."""
    s = (amax / F32(E4M3_MAX)).astype(F32)
    safe = np.where(s > 0, s, F32(1.0)).astype(F32)
    q = e4m3_encode((vals / safe).astype(F32))
    q = np.where(s > 0, q, np.uint8(0)).astype(np.uint8)
    return s, q


def quant_fp8(h_bits: np.ndarray) -> Dict[str, np.ndarray]:
    """Row (1x128) and transposed (128x128 block) e4m3 quantization of bf16 h [M, F]."""
    h = bf16_to_f32(np.asarray(h_bits))
    M, F = h.shape
    if F % TILE != 0:
        raise ValueError("F must be a multiple of 128")
    nt = F // TILE
    m_pad = -(-M // TILE) * TILE
    nb = m_pad // TILE

    # row layout: one scale per (row, 128-column tile)
    ht = h.reshape(M, nt, TILE)
    amax_row = np.abs(ht).max(axis=2, initial=F32(0)).astype(F32)          # [M, nt]
    s_row, q_row = _tile_codes(ht, amax_row[:, :, None])
    q_row = q_row.reshape(M, F)
    s_row = s_row.reshape(M, nt)

    # transposed layout: one scale per 128x128 block over real rows
    q_t = np.zeros((F, m_pad), dtype=np.uint8)
    s_t = np.zeros((nt, nb), dtype=F32)
    for mb in range(nb):
        r0, r1 = mb * TILE, min(M, (mb + 1) * TILE)
        for fb in range(nt):
            blk = h[r0:r1, fb * TILE:(fb + 1) * TILE]
            amax = np.abs(blk).max(initial=F32(0)).astype(F32)
            s, q = _tile_codes(blk, amax)
            s_t[fb, mb] = s
            q_t[fb * TILE:(fb + 1) * TILE, r0:r1] = q.T
    return {"q_row": q_row, "s_row": s_row, "q_t": q_t, "s_t": s_t}


def swiglu_quant_fp8(gate_up_bits: np.ndarray, F: int) -> Dict[str, np.ndarray]:
    """quant_fp8(swiglu(x)) on x [M, 2F] (gate columns first); also returns h."""
    h = swiglu(gate_up_bits, F)
    res = quant_fp8(h)
    res["h"] = h
    return res


def expand_128x_starts(group_sizes) -> tuple:
    """First q_t column of each group in the expanded layout, and the padded total."""
    padded = [-(-int(n) // TILE) * TILE for n in group_sizes]
    starts, acc = [], 0
    for p in padded:
        starts.append(acc)
        acc += p
    return starts, acc


def quant_fp8_grouped(h_bits: np.ndarray, group_sizes=None, trans: str = "block",
                      m_pad=None) -> Dict[str, np.ndarray]:
    """Row layout (1x128 tiles) and the grouped, expand_128x transposed layout of bf16 h [M, K].

    group_sizes: row counts of consecutive groups summing to M (None: one
    group of M rows). trans: "block" (one scale per 128x128 block) or "tile"
    (one scale per column and 128-row tile). m_pad: width of q_t, a multiple
    of 128 no smaller than the groups' padded total (None: that total).
    """
    h = bf16_to_f32(np.asarray(h_bits))
    M, K = h.shape
    if K % TILE != 0:
        raise ValueError("K must be a multiple of 128")
    if trans not in ("block", "tile"):
        raise ValueError("trans must be 'block' or 'tile'")
    sizes = [M] if group_sizes is None else [int(n) for n in group_sizes]
    if any(n < 0 for n in sizes) or sum(sizes) != M:
        raise ValueError("group sizes must be non-negative and sum to M")
    starts, total = expand_128x_starts(sizes)
    m_pad = total if m_pad is None else int(m_pad)
    if m_pad < total or m_pad % TILE != 0:
        raise ValueError("m_pad must be a multiple of 128 covering every group's padded rows")
    nt = K // TILE

    # row layout: as quant_fp8, independent of the groups
    ht = h.reshape(M, nt, TILE)
    amax_row = np.abs(ht).max(axis=2, initial=F32(0)).astype(F32)
    s_row, q_row = _tile_codes(ht, amax_row[:, :, None])

    q_t = np.zeros((K, m_pad), dtype=np.uint8)
    s_t = np.zeros((nt if trans == "block" else K, m_pad // TILE), dtype=F32)
    row0 = 0
    for n, col0 in zip(sizes, starts):
        for j in range(-(-n // TILE)):
            r0, r1 = row0 + j * TILE, min(row0 + n, row0 + (j + 1) * TILE)
            c0 = col0 + j * TILE
            tile = h[r0:r1]                                             # [rows, K]
            if trans == "block":
                for fb in range(nt):
                    blk = tile[:, fb * TILE:(fb + 1) * TILE]
                    s, q = _tile_codes(blk, np.abs(blk).max(initial=F32(0)).astype(F32))
                    s_t[fb, c0 // TILE] = s
                    q_t[fb * TILE:(fb + 1) * TILE, c0:c0 + (r1 - r0)] = q.T
            else:
                amax_col = np.abs(tile).max(axis=0, initial=F32(0)).astype(F32)    # [K]
                s, q = _tile_codes(tile, amax_col[None, :])
                s_t[:, c0 // TILE] = s
                q_t[:, c0:c0 + (r1 - r0)] = q.T
        row0 += n
    return {"q_row": q_row.reshape(M, K), "s_row": s_row.reshape(M, nt), "q_t": q_t, "s_t": s_t}


def block_quant_fp8(w_bits: np.ndarray) -> Dict[str, np.ndarray]:
    """e4m3 quantization of a bf16 weight matrix [N, K] with one scale per
    128x128 block, kept in the weight's own row-major layout: q [N, K] uint8,
    s [N/128, K/128] float32, s = fl32(amax/448), code = e4m3(fl32(w/s)).

    The FP8 grouped-GEMM item of the MoE path pairs the 1x128-tile activation
    codes with "128x128-block-scaled e4m3 weights"; a block of the weight is
    quantized exactly as a block of the transposed activation layout is.
    """
    w = bf16_to_f32(np.asarray(w_bits))
    N, K = w.shape
    if N % TILE or K % TILE:
        raise ValueError("N and K must be multiples of 128")
    blocks = w.reshape(N // TILE, TILE, K // TILE, TILE)
    amax = np.abs(blocks).max(axis=(1, 3), initial=F32(0)).astype(F32)       # [N/128, K/128]
    s, q = _tile_codes(blocks, amax[:, None, :, None])
    return {"q": q.reshape(N, K), "s": s.reshape(N // TILE, K // TILE)}


def grouped_gemm_fp8(qa: np.ndarray, sa: np.ndarray, qw: np.ndarray, sw: np.ndarray,
                     group_sizes: np.ndarray, group_offsets: np.ndarray) -> np.ndarray:
    """y[e] = bf16(A_e @ W_e^T) on block-scaled e4m3 operands, in float64:
    A [numel, K] codes qa with one scale per row and 128-column tile sa
    [numel, K/128] (the quantizer's row layout); W_e [N, K] codes qw[e] with
    one scale per 128x128 block sw[e] [N/128, K/128]. Each operand is its
    decoded code times its scale; returns uint16 bf16 bits [numel, N].
    """
    E, N, K = qw.shape
    numel = qa.shape[0]
    out = np.zeros((numel, N), dtype=np.uint16)
    a_all = e4m3_decode(np.asarray(qa)).astype(np.float64) * np.repeat(np.asarray(sa, np.float64), TILE, axis=1)
    for e in range(E):
        n = int(group_sizes[e])
        if n == 0:
            continue
        o = int(group_offsets[e])
        wdec = e4m3_decode(np.asarray(qw[e])).astype(np.float64)
        wscale = np.repeat(np.repeat(np.asarray(sw[e], np.float64), TILE, axis=0), TILE, axis=1)
        out[o:o + n] = to_bf16(a_all[o:o + n] @ (wdec * wscale).T)
    return out
