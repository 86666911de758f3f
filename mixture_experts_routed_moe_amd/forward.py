"""The routed-expert MoE forward as a sequence of library calls.

Stage order follows the TileOPs routed pipeline (#1580, "Grouped-GEMM
kernel" and "Unpermute"; #778, "Partial output contract" for the shared
expert): routing, dispatch tables, permute, gate_up GEMM (+ SwiGLU), down
GEMM, unpermute with the routing weights and routed_scaling_factor folded in
before the store. The shared expert, when given, runs the same two GEMMs on
all tokens as one dense group and joins the unpermute as its addend. By
default the permute is folded into the gate_up GEMM, which reads each
permuted row from the hidden states through the dispatch permutation
(`grouped_gemm_gate_up_gather`); `fuse_permute=False` runs it as its own
copy first.

`MoEBuffers` holds every intermediate for one problem size so a forward
allocates nothing; all work is enqueued on the current stream without a host
synchronisation. Given `shared_stream`, the shared expert's two GEMMs run on
that stream instead, concurrently with routing, permute and the routed GEMMs
(they depend only on the hidden states), and the current stream waits for
them before the unpermute: the routed kernels leave matrix cores idle while
they wait on weight loads, and the shared expert's dense tiles fill them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

from . import _lib


@dataclasses.dataclass
class MoEShape:
    T: int
    H: int
    F: int
    E: int
    top_k: int
    padding_m: int = 128
    block_m: int = 128
    shared_F: int = 0

    @property
    def numel(self) -> int:
        return self.T * self.top_k


class MoEBuffers:
    """Device buffers for every intermediate of one forward of `shape`."""

    def __init__(self, shape: MoEShape, device, fuse_swiglu: bool = True, fuse_permute: bool = True,
                 fp8_down: bool = False, fp8_gate_up: bool = False, fp8_shared: bool = False):
        s = shape
        self.shape = s
        self.fuse_swiglu = fuse_swiglu
        self.fuse_permute = fuse_permute
        self.fp8_down = fp8_down
        self.fp8_gate_up = fp8_gate_up
        self.fp8_shared = fp8_shared
        bf16 = dict(dtype=torch.bfloat16, device=device)
        self.topk_ids = torch.empty(s.T, s.top_k, dtype=torch.int32, device=device)
        self.topk_weights = torch.empty(s.T, s.top_k, dtype=torch.float32, device=device)
        self.tables = _lib.alloc_tables(s.numel, s.E, s.padding_m, s.block_m, device)
        # the permuted copy of the hidden states exists only without the gather
        self.x_perm = None if fuse_permute else torch.empty(s.numel, s.H, **bf16)
        self.gate_up = None if fuse_swiglu else torch.empty(s.numel, 2 * s.F, **bf16)
        self.h = torch.empty(s.numel, s.F, **bf16)
        self.y = torch.empty(s.numel, s.H, **bf16)
        # e4m3 codes of h and their 1x128-tile scales, for the FP8 down projection
        self.qa = None if not fp8_down else {
            "q_row": torch.empty(s.numel, s.F, dtype=torch.uint8, device=device),
            "s_row": torch.empty(s.numel, s.F // 128, dtype=torch.float32, device=device)}
        # e4m3 codes of the hidden states (one row per token), for the FP8 gate_up GEMMs
        self.qh = None if not (fp8_gate_up or fp8_shared) else {
            "q_row": torch.empty(s.T, s.H, dtype=torch.uint8, device=device),
            "s_row": torch.empty(s.T, s.H // 128, dtype=torch.float32, device=device)}
        self.out = torch.empty(s.T, s.H, **bf16)
        # e4m3 codes of the shared expert's h, for its FP8 down projection
        self.qsh = None if not (fp8_shared and s.shared_F) else {
            "q_row": torch.empty(s.T, s.shared_F, dtype=torch.uint8, device=device),
            "s_row": torch.empty(s.T, s.shared_F // 128, dtype=torch.float32, device=device)}
        if s.shared_F:
            self.shared_gate_up = None if fuse_swiglu else torch.empty(s.T, 2 * s.shared_F, **bf16)
            self.shared_h = torch.empty(s.T, s.shared_F, **bf16)
            self.shared_y = torch.empty(s.T, s.H, **bf16)


def routed_moe_forward(hidden: torch.Tensor, router_logits: torch.Tensor, w_gate_up: torch.Tensor,
                       w_down: torch.Tensor, top_k: int, routed_scaling_factor: float = 1.0,
                       padding_m: int = 128, block_m: int = 128,
                       shared_w_gate_up: Optional[torch.Tensor] = None,
                       shared_w_down: Optional[torch.Tensor] = None,
                       fuse_swiglu: bool = True, buffers: Optional[MoEBuffers] = None,
                       expert_bias: Optional[torch.Tensor] = None, scoring: str = "softmax",
                       renormalize: bool = True, return_parts: bool = False,
                       shared_stream: Optional[torch.cuda.Stream] = None, fuse_permute: bool = True,
                       w_down_fp8: Optional[Dict[str, torch.Tensor]] = None,
                       w_gate_up_fp8: Optional[Dict[str, torch.Tensor]] = None,
                       w_shared_fp8: Optional[Dict[str, Dict[str, torch.Tensor]]] = None):
    """out [T, H] bf16 = rsf * sum_j w_j * expert_j(hidden) (+ shared_expert(hidden)).

    With return_parts=True returns (shared_out, routed_out) instead, the split
    of TileOPs #778 "Partial output contract": shared_out [T, H] bf16 (None
    without a shared expert) and routed_out the routed sum alone; the caller
    adds them (after its all-reduce of shared_out when the shared expert is
    tensor-parallel). Otherwise the shared output is added inside the
    unpermute before its single rounding.

    w_down_fp8: the routed down projection in FP8: {"q", "s"} from
    fp8_block_quant_weights(w_down) (e4m3 codes [E, H, F], one scale per
    128x128 block); h is quantized to 1x128-tile e4m3 codes (row layout) and
    grouped_gemm_fp8 replaces the bf16 down GEMM (block_m 128; buffers made
    with fp8_down=True). The shared expert stays bf16.

    w_gate_up_fp8: the routed gate_up in FP8: {"q", "s"} from
    fp8_block_quant_weights(w_gate_up); the hidden states are quantized once
    per token to 1x128-tile e4m3 codes and grouped_gemm_gate_up_fp8 reads each
    pair's row through the dispatch permutation (needs fuse_permute; buffers
    made with fp8_gate_up=True).

    w_shared_fp8: the shared expert's two GEMMs in FP8: {"gate_up": ...,
    "down": ...}, each from fp8_block_quant_weights of the shared weights; its
    gate_up reads the hidden states' e4m3 codes (one dense group), its h is
    quantized to 1x128-tile codes for the down projection (buffers made with
    fp8_shared=True; block_m 128).

    fuse_permute: the gate_up GEMM reads each permuted row straight from
    `hidden` (row sorted_pair[r] // top_k) instead of a permuted copy written
    by moe_permute: the same bytes, without the copy's write and re-read.

    shared_stream: a stream (of default priority) for the shared expert's
    GEMMs; it first waits for the work already on the current stream, and
    the current stream waits for it before the unpermute (and before
    returning with return_parts). The results are the same bits either way.
    """
    T, H = hidden.shape
    E, twoF, H2 = w_gate_up.shape
    F = twoF // 2
    if H2 != H or tuple(w_down.shape) != (E, H, F) or tuple(router_logits.shape) != (T, E):
        raise ValueError("routed_moe_forward: inconsistent shapes")
    shared_F = 0 if shared_w_down is None else shared_w_down.shape[1]
    shape = MoEShape(T, H, F, E, top_k, padding_m, block_m, shared_F)
    b = buffers
    if b is None:
        b = MoEBuffers(shape, hidden.device, fuse_swiglu, fuse_permute, w_down_fp8 is not None,
                       w_gate_up_fp8 is not None, w_shared_fp8 is not None)
    elif (dataclasses.astuple(b.shape) != dataclasses.astuple(shape) or b.fuse_swiglu != fuse_swiglu
          or b.fuse_permute != fuse_permute or (w_down_fp8 is not None and b.qa is None)
          or (w_gate_up_fp8 is not None and b.qh is None)
          or (w_shared_fp8 is not None and shared_F and b.qsh is None)):
        raise ValueError("routed_moe_forward: buffers were made for another shape")

    quant_hidden = w_gate_up_fp8 is not None or (w_shared_fp8 is not None and shared_F)
    if quant_hidden:
        # the hidden states' e4m3 codes, read by both FP8 gate_up GEMMs
        _lib.tile_quant_fp8(hidden, out=b.qh, transposed=False)

    def shared_expert():
        sgu = b.shared_h if fuse_swiglu else b.shared_gate_up
        if w_shared_fp8 is not None:
            _lib.grouped_gemm_gate_up_fp8(b.qh["q_row"], b.qh["s_row"], w_shared_fp8["gate_up"]["q"],
                                          w_shared_fp8["gate_up"]["s"], None, padding_m, block_m, fuse_swiglu,
                                          out=sgu)
        else:
            _lib.grouped_gemm_gate_up(hidden, shared_w_gate_up, None, padding_m, block_m, fuse_swiglu, sgu)
        if not fuse_swiglu:
            _lib.swiglu(b.shared_gate_up, b.shared_h)
        if w_shared_fp8 is not None:
            _lib.tile_quant_fp8(b.shared_h, out=b.qsh, transposed=False)
            _lib.grouped_gemm_fp8(b.qsh["q_row"], b.qsh["s_row"], w_shared_fp8["down"]["q"],
                                  w_shared_fp8["down"]["s"], None, padding_m, block_m, b.shared_y)
        else:
            _lib.grouped_gemm_down(b.shared_h, shared_w_down, None, padding_m, block_m, b.shared_y)

    main = torch.cuda.current_stream(hidden.device)
    side = shared_stream if shared_F else None
    if side is not None:
        side.wait_stream(main)
        with torch.cuda.stream(side):
            shared_expert()
    _lib.moe_topk_softmax(router_logits, top_k, b.topk_ids, b.topk_weights, expert_bias, scoring, renormalize)
    tb = _lib.moe_align(b.topk_ids, E, padding_m, block_m, b.tables)
    gu_out = b.h if fuse_swiglu else b.gate_up
    if w_gate_up_fp8 is not None:
        if not fuse_permute:
            raise ValueError("routed_moe_forward: the FP8 gate_up reads its rows through the permutation "
                             "(fuse_permute=True)")
        _lib.grouped_gemm_gate_up_fp8(b.qh["q_row"], b.qh["s_row"], w_gate_up_fp8["q"], w_gate_up_fp8["s"], tb,
                                      padding_m, block_m, fuse_swiglu, top_k=top_k, out=gu_out)
    elif fuse_permute:
        _lib.grouped_gemm_gate_up_gather(hidden, w_gate_up, tb, top_k, padding_m, block_m, fuse_swiglu, gu_out)
    else:
        _lib.moe_permute(hidden, tb["sorted_pair"], top_k, b.x_perm, tb["pair_to_row"])
        _lib.grouped_gemm_gate_up(b.x_perm, w_gate_up, tb, padding_m, block_m, fuse_swiglu, gu_out)
    if not fuse_swiglu:
        _lib.swiglu(b.gate_up, b.h)
    if w_down_fp8 is None:
        _lib.grouped_gemm_down(b.h, w_down, tb, padding_m, block_m, b.y)
    else:
        _lib.tile_quant_fp8(b.h, out=b.qa, transposed=False)
        _lib.grouped_gemm_fp8(b.qa["q_row"], b.qa["s_row"], w_down_fp8["q"], w_down_fp8["s"], tb, padding_m,
                              block_m, b.y)
    addend = None
    if shared_F:
        if side is None:
            shared_expert()
        else:
            main.wait_stream(side)
        addend = b.shared_y
    if return_parts:
        _lib.moe_unpermute(b.y, tb["pair_to_row"], b.topk_weights, routed_scaling_factor, None, b.out)
        return addend, b.out
    _lib.moe_unpermute(b.y, tb["pair_to_row"], b.topk_weights, routed_scaling_factor, addend, b.out)
    return b.out


class MoEForwardGraph:
    """One forward captured as a HIP graph over static input tensors.

    The library's calls allocate nothing, wait on nothing from the host and
    issue no memset or copy, so with reusable buffers a forward is a fixed
    sequence of kernel launches (plus, with `shared_stream`, a fork to that
    stream and a join back) and captures whole. Replaying it costs one graph
    launch instead of one host call per kernel, which is what the forward of a
    few decode tokens is bound by. Write new inputs into `.hidden` and
    `.logits` (in place), call `replay()`, read `.out`; the weights, the expert
    bias and every other argument are fixed at capture. Replays are ordered on
    the stream current at `replay()`.
    """

    def __init__(self, hidden: torch.Tensor, router_logits: torch.Tensor, w_gate_up: torch.Tensor,
                 w_down: torch.Tensor, top_k: int, routed_scaling_factor: float = 1.0, padding_m: int = 128,
                 block_m: int = 128, shared_w_gate_up: Optional[torch.Tensor] = None,
                 shared_w_down: Optional[torch.Tensor] = None, fuse_swiglu: bool = True,
                 buffers: Optional[MoEBuffers] = None, expert_bias: Optional[torch.Tensor] = None,
                 scoring: str = "softmax", renormalize: bool = True,
                 shared_stream: Optional[torch.cuda.Stream] = None, fuse_permute: bool = True,
                 w_down_fp8: Optional[Dict[str, torch.Tensor]] = None,
                 w_gate_up_fp8: Optional[Dict[str, torch.Tensor]] = None,
                 w_shared_fp8: Optional[Dict[str, Dict[str, torch.Tensor]]] = None):
        T, H = hidden.shape
        E, twoF, _ = w_gate_up.shape
        shared_F = 0 if shared_w_down is None else shared_w_down.shape[1]
        if buffers is None:
            buffers = MoEBuffers(MoEShape(T, H, twoF // 2, E, top_k, padding_m, block_m, shared_F), hidden.device,
                                 fuse_swiglu, fuse_permute, w_down_fp8 is not None, w_gate_up_fp8 is not None,
                                 w_shared_fp8 is not None)
        self.hidden, self.logits, self.buffers = hidden, router_logits, buffers

        def run():
            return routed_moe_forward(hidden, router_logits, w_gate_up, w_down, top_k, routed_scaling_factor,
                                      padding_m, block_m, shared_w_gate_up, shared_w_down, fuse_swiglu, buffers,
                                      expert_bias, scoring, renormalize, shared_stream=shared_stream,
                                      fuse_permute=fuse_permute, w_down_fp8=w_down_fp8,
                                      w_gate_up_fp8=w_gate_up_fp8, w_shared_fp8=w_shared_fp8)

        # one eager forward first: loads the library and checks every argument
        run()
        torch.cuda.current_stream(hidden.device).synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out = run()

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.out


def intermediates(b: MoEBuffers) -> Dict[str, torch.Tensor]:
    d = {"topk_ids": b.topk_ids, "topk_weights": b.topk_weights, "h": b.h, "y": b.y, "out": b.out}
    if b.x_perm is not None:
        d["x_perm"] = b.x_perm
    d.update({k: v for k, v in b.tables.items() if k != "workspace"})
    if b.gate_up is not None:
        d["gate_up"] = b.gate_up
    if b.shape.shared_F:
        d["shared"] = b.shared_y
    return d
