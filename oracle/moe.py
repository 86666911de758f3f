"""Oracle for the routed-expert MoE forward: a plain, slow host implementation.

Test infrastructure only (see oracle/__init__.py). Each function restates one
step as the pages define it, in the order they give:

  route             router logits (+ bias) scored by softmax or sigmoid, top-k, weights
                    renormalised or not
  dispatch_tables   group_sizes / group_offsets / group_padded_offsets /
                    group_idx_for_bx and the expert-major permutation
  block_decode      the kernel-side row recovery of one row block
  permute           gather token rows into the compact expert-major layout
  grouped_gemm      C[e] = A[e] @ B[e]^T per expert, B stored [N, K]
  swiglu            SiLU(gate) * up on the gate|up halves
  unpermute         weighted sum over the k slots, routed_scaling_factor
                    applied before the single rounding, optional addend
  shared_expert     the dense SwiGLU MLP of the shared expert
  forward           the whole path

Precision: matrix products and weighted sums are taken in float64 (products
of bf16 values are exact there) and rounded once to bf16 wherever the method
stores a bf16 tensor. Routing weights are formed in float64 and stored as
float32. The SwiGLU follows the fp32 specification in numerics.py because an
FP8 code downstream depends on its exact bits.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .numerics import bf16_to_f32, bf16_to_f64, silu32, to_bf16


# ------------------------------------------------------------------ route --

def route(logits: np.ndarray, top_k: int, bias: Optional[np.ndarray] = None, scoring: str = "softmax",
          renormalize: bool = True):
    """Top-k routing.

    The op's routing input is a [T, E] score tensor ("gating" in the call of
    TileOPs #778, "Partial output contract"); the tutorial's example routes
    every token to top_k experts ("Example 07 ... expected output"). The
    workload description fixes softmax -> top-k -> renormalise; TileOPs #778's
    Kimi-K2 benchmark names sigmoid routing.

    Routing logit v = logits + bias, one float32 addition (bias is the
    per-expert skew of the DeepSeek-V3-shaped workload; the pages give no
    formula, so it enters selection and scoring alike). Selection: experts
    ordered by descending v, ties to the lower expert id; slot j holds the
    j-th expert of that order. Scores, in float64: softmax of v over all E,
    or the logistic sigmoid of each v. Weights: the selected scores divided by
    their sum (renormalize) or the scores themselves; stored as float32.
    """
    v = np.asarray(logits, dtype=np.float32)
    T, E = v.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k out of range")
    if bias is not None:
        v = (v + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    # stable argsort of -v: equal logits keep ascending expert id
    order = np.argsort(-v, axis=1, kind="stable")
    ids = order[:, :top_k].astype(np.int32)
    v64 = v.astype(np.float64)
    if scoring == "softmax":
        ex = np.exp(v64 - v64.max(axis=1, keepdims=True))
        p = ex / ex.sum(axis=1, keepdims=True)
    elif scoring == "sigmoid":
        p = 1.0 / (1.0 + np.exp(-v64))
    else:
        raise ValueError("scoring must be 'softmax' or 'sigmoid'")
    p_sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        p_sel = p_sel / p_sel.sum(axis=1, keepdims=True)
    return ids, p_sel.astype(np.float32)


# -------------------------------------------------------- dispatch tables --

def num_blocks(numel: int, E: int, block_m: int, padding_m: int) -> int:
    """Upper bound on padded row blocks: ceil(numel / block_m) + E * (padding_m / block_m).

    Tutorial Example 07, expected output: 18 pairs, 4 experts, 128-row blocks
    and 128-row padding give 5 = ceil(18/128) + 4 blocks. The page always has
    padding_m == block_m; when padding_m is a larger multiple c of block_m,
    each expert's rounding can add up to c blocks, so E is counted c times
    (the same formula when c = 1).
    """
    return -(-numel // block_m) + E * (padding_m // block_m)


def dispatch_tables(topk_ids: np.ndarray, E: int, padding_m: int, block_m: int) -> Dict[str, object]:
    """The four host tables of the dispatch contract plus the permutation.

    Tutorial Example 07 ("moe_dispatch_contract.py", purpose and expected
    output) defines, over the T*k (token, expert) pairs:
      group_sizes[e]          pairs routed to expert e
      group_offsets[e]        start of e's rows in the compact layout
                              (exclusive prefix sum of the sizes)
      group_padded_offsets[e] start of e's range once every group is rounded
                              up to a multiple of padding_m
      group_idx_for_bx[bx]    the expert owning padded row block bx, found by
                              a linear scan (the tutorial notes a real
                              framework may vectorise it)
    Readings where the page is silent: an empty expert pads to 0 rows and an
    exact multiple is not padded further (ceil(s/P)*P); block bx belongs to the
    last expert whose padded offset is <= bx*block_m, so empty experts are
    passed over and surplus blocks land on the last expert; inside an expert,
    rows keep ascending pair order (pair p = t*k + j), i.e. a stable counting
    sort by expert id.
    """
    ids = np.asarray(topk_ids).reshape(-1)
    numel = ids.size
    if padding_m <= 0 or block_m <= 0 or padding_m % block_m != 0:
        raise ValueError("padding_m must be a positive multiple of block_m")
    ids_list = [int(x) for x in ids]
    for x in ids_list:
        if not (0 <= x < E):
            raise ValueError("expert id out of range")

    sizes = [0] * E
    for e in ids_list:
        sizes[e] += 1
    offsets = [0] * E
    padded = [0] * E
    acc = 0
    pacc = 0
    for e in range(E):
        offsets[e] = acc
        padded[e] = pacc
        acc += sizes[e]
        pacc += -(-sizes[e] // padding_m) * padding_m
    m_blocks = num_blocks(numel, E, block_m, padding_m)

    gidx = [0] * m_blocks
    for bx in range(m_blocks):
        g = 0
        for cand in range(E):                      # linear scan, last match wins
            if padded[cand] <= bx * block_m:
                g = cand
        gidx[bx] = g

    cursor = list(offsets)
    sorted_pair = [0] * numel
    for p, e in enumerate(ids_list):
        sorted_pair[cursor[e]] = p
        cursor[e] += 1
    pair_to_row = [0] * numel
    for r, p in enumerate(sorted_pair):
        pair_to_row[p] = r

    i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return {
        "group_sizes": i32(sizes),
        "group_offsets": i32(offsets),
        "group_padded_offsets": i32(padded),
        "group_idx_for_bx": i32(gidx),
        "sorted_pair": i32(sorted_pair),
        "pair_to_row": i32(pair_to_row),
        "m_blocks": m_blocks,
        "group_sum": numel,
        "padded_total": pacc,
        "waste": m_blocks * block_m - numel,
    }


def block_decode(tables: Dict[str, object], bx: int, block_m: int):
    """Kernel-side row recovery for padded row block bx -> (g, m_start, actual_rows).

    Tutorial Example 07, purpose item 4:
      m_start = m_start_padded - group_padded_offsets[g] + group_offsets[g]
    with m_start_padded = bx*block_m. actual_rows is the number of rows of
    the block that hold pairs of g (the masked partial tile of TileOPs #1580,
    "Grouped-GEMM kernel"): clamp(offset + size - m_start, 0, block_m).
    """
    g = int(tables["group_idx_for_bx"][bx])
    gs = int(tables["group_sizes"][g])
    go = int(tables["group_offsets"][g])
    gpo = int(tables["group_padded_offsets"][g])
    m_start = bx * block_m - gpo + go
    actual = min(max(go + gs - m_start, 0), block_m)
    return g, m_start, actual


# ------------------------------------------------------- permute / GEMM --

def permute(hidden_bits: np.ndarray, sorted_pair: np.ndarray, top_k: int) -> np.ndarray:
    """x_perm[r] = hidden[sorted_pair[r] // top_k] (bf16 bit copy)."""
    return np.asarray(hidden_bits)[np.asarray(sorted_pair, dtype=np.int64) // top_k].copy()


def grouped_gemm(a_bits: np.ndarray, w_bits: np.ndarray, group_sizes: np.ndarray,
                 group_offsets: np.ndarray) -> np.ndarray:
    """C[e] = A[e] @ B[e]^T for every expert with rows; B[e] is stored [N, K].

    TileOPs #1580 ("Benchmark results") states the grouped GEMM as
    C[e] = A[e] @ B[e]^T; A is the compact (numel, K) layout ("Grouped-GEMM
    kernel": A_shape = (numel, K)). Each output is the float64 product
    rounded once to bf16. Returns uint16 [numel, N].
    """
    a = np.asarray(a_bits)
    w = np.asarray(w_bits)
    numel = a.shape[0]
    N = w.shape[1]
    out = np.zeros((numel, N), dtype=np.uint16)
    for e in range(w.shape[0]):
        s = int(group_sizes[e])
        if s == 0:
            continue
        o = int(group_offsets[e])
        acc = bf16_to_f64(a[o:o + s]) @ bf16_to_f64(w[e]).T
        out[o:o + s] = to_bf16(acc)
    return out


def swiglu(gate_up_bits: np.ndarray, F: int) -> np.ndarray:
    """h = bf16(silu32(gate) * up) on [M, 2F] -> [M, F] (gate = columns 0..F-1).

    SiLU(gate) * up is the activation between the two GEMMs (TileOPs #778,
    "New files": gate+up GEMM, SiLU-mul, down GEMM; xtuner #2089, "Changes":
    SiLU(gate) * up). The fp32 product is rounded to bf16, the precision the
    unfused activation stores (xtuner #2089: native_swiglu gives bf16).
    """
    gu = np.asarray(gate_up_bits)
    g = bf16_to_f32(gu[:, :F])
    u = bf16_to_f32(gu[:, F:2 * F])
    return to_bf16((silu32(g) * u).astype(np.float32))


def unpermute(y_bits: np.ndarray, pair_to_row: np.ndarray, topk_weights: np.ndarray,
              top_k: int, routed_scaling_factor: float,
              addend_bits: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = bf16(rsf * sum_j w[t,j] * y[pair_to_row[t*k+j]] (+ addend[t])).

    TileOPs #1580 ("Unpermute"): the weighted sum over the k expert outputs
    of a token, with routed_scaling_factor applied before the cast and store.
    The sum runs over j ascending in float64; rsf is the float32 value the
    kernel receives. The optional addend (the shared expert's output) joins
    before the single rounding.
    """
    y = bf16_to_f64(y_bits)
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T = w.shape[0]
    rows = np.asarray(pair_to_row, dtype=np.int64).reshape(T, top_k)
    acc = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(top_k):
        acc += w[:, j:j + 1] * y[rows[:, j]]
    rsf = float(np.float32(routed_scaling_factor))
    val = rsf * acc
    if addend_bits is not None:
        val = val + bf16_to_f64(addend_bits)
    return to_bf16(val)


def shared_expert(hidden_bits: np.ndarray, w_gate_up_bits: np.ndarray,
                  w_down_bits: np.ndarray) -> np.ndarray:
    """Dense SwiGLU MLP: bf16(swiglu(bf16(x @ Wgu^T)) @ Wd^T).

    TileOPs #778 ("New files", "Modified files"): gate+up GEMM with
    w_gate_up [2F_s, H], SiLU-mul, down GEMM with w_down [H, F_s]. It is the
    grouped path with a single group holding every token.
    """
    T = hidden_bits.shape[0]
    one = np.array([T], dtype=np.int32)
    zero = np.array([0], dtype=np.int32)
    F_s = w_down_bits.shape[1]
    gu = grouped_gemm(hidden_bits, w_gate_up_bits[None], one, zero)
    h = swiglu(gu, F_s)
    return grouped_gemm(h, w_down_bits[None], one, zero)


def forward(hidden_bits: np.ndarray, logits: np.ndarray, w_gate_up_bits: np.ndarray,
            w_down_bits: np.ndarray, top_k: int, routed_scaling_factor: float = 1.0,
            padding_m: int = 128, block_m: int = 128,
            shared_w_gate_up_bits: Optional[np.ndarray] = None,
            shared_w_down_bits: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None,
            scoring: str = "softmax", renormalize: bool = True) -> Dict[str, np.ndarray]:
    """The whole routed (+ shared) forward; returns every intermediate.

    Order as the TileOPs pipeline runs it (#1580 "Grouped-GEMM kernel" and
    "Unpermute"; #778 "Partial output contract" for the shared part):
    route, tables, permute, gate_up GEMM, SwiGLU, down GEMM, unpermute; the
    shared expert's output is added to the routed output.
    """
    E, twoF, H = w_gate_up_bits.shape
    F = twoF // 2
    ids, w = route(logits, top_k, bias, scoring, renormalize)
    tab = dispatch_tables(ids, E, padding_m, block_m)
    x_perm = permute(hidden_bits, tab["sorted_pair"], top_k)
    gu = grouped_gemm(x_perm, w_gate_up_bits, tab["group_sizes"], tab["group_offsets"])
    h = swiglu(gu, F)
    y = grouped_gemm(h, w_down_bits, tab["group_sizes"], tab["group_offsets"])
    shared = None
    if shared_w_gate_up_bits is not None:
        shared = shared_expert(hidden_bits, shared_w_gate_up_bits, shared_w_down_bits)
    out = unpermute(y, tab["pair_to_row"], w, top_k, routed_scaling_factor, shared)
    res = dict(tab)
    res.update(topk_ids=ids, topk_weights=w, x_perm=x_perm, gate_up=gu, h=h, y=y, out=out)
    if shared is not None:
        res["shared"] = shared
    return res

