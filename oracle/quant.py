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
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .moe import swiglu
from .numerics import E4M3_MAX, bf16_to_f32, e4m3_encode

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
