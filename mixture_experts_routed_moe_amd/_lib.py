"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Each function takes torch tensors that live on the GPU, checks dtype, shape
and contiguity, passes raw device pointers and the current HIP stream to the
C entry point of the same name, and raises MoeError on a non-zero return.
Every computation happens in the library's HIP kernels; there is no host or
PyTorch fallback: the first call raises ImportError if the library is missing
or was built for another ABI revision (the import itself does not load it, so
the build step can run from a fresh checkout).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


ABI_VERSION = 8
SCORING = {"softmax": 0, "sigmoid": 1}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mixture_experts_routed_moe_amd.build` "
            "(the MoE path has no fallback without its HIP library)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (I, []),
        "moe_num_blocks": (I64, [I64, I, I, I]),
        "moe_align_workspace_bytes": (SZ, [I64, I]),
        "moe_topk_softmax": (I, [P, P, I64, I, I, I, I, P, P, P]),
        "moe_align": (I, [P, I64, I, I, I, I, P, P, P, P, P, P, P, SZ, P]),
        "moe_align_noalloc": (I, [P, I64, I, I, I, I, P, P, P, P, P, P, P]),
        "moe_align_noalloc_max_scratch_bytes": (SZ, []),
        "moe_permute": (I, [P, P, P, I64, I, I, P, P]),
        "grouped_gemm_gate_up": (I, [P, P, P, P, P, P, I64, I, I, I, I, I, I, P, P]),
        "grouped_gemm_gate_up_gather": (I, [P, I64, P, I, P, P, P, P, P, I64, I, I, I, I, I, I, P, P]),
        "swiglu": (I, [P, I64, I, P, P]),
        "grouped_gemm_down": (I, [P, P, P, P, P, P, I64, I, I, I, I, I, P, P]),
        "moe_unpermute": (I, [P, P, P, I64, I, I, F, P, P, P]),
        "swiglu_quant_fp8": (I, [P, I64, I, P, P, P, P, P]),
        "tile_quant_fp8": (I, [P, I64, I, I, P, I, I, I64, P, P, P, P, P]),
        "tile_quant_fp8_m_pad_bound": (I64, [I64, I]),
        "fp8_block_quant_weights": (I, [P, I64, I, P, P, P]),
        "grouped_gemm_fp8": (I, [P, P, P, P, P, P, P, P, I64, I, I, I, I, I, P, P]),
        "grouped_gemm_gate_up_fp8": (I, [P, P, I64, P, I, P, P, P, P, P, P, I64, I, I, I, I, I, I, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI {lib.moe_abi_version()}, this binding needs {ABI_VERSION}: rebuild it "
                          "with `python -m mixture_experts_routed_moe_amd.build`")
    return lib


_lib: Optional[ctypes.CDLL] = None

EXPORTS = ("moe_last_error", "moe_abi_version", "moe_num_blocks", "moe_align_workspace_bytes",
           "moe_topk_softmax", "moe_align", "moe_permute", "grouped_gemm_gate_up",
           "grouped_gemm_gate_up_gather", "swiglu",
           "grouped_gemm_down", "moe_unpermute", "swiglu_quant_fp8", "tile_quant_fp8",
           "tile_quant_fp8_m_pad_bound", "fp8_block_quant_weights", "grouped_gemm_fp8", "grouped_gemm_gate_up_fp8",
           "moe_align_noalloc", "moe_align_noalloc_max_scratch_bytes")


def lib() -> ctypes.CDLL:
    """The loaded library; loads it on first use and raises ImportError when
    it is missing or was built for another ABI revision (there is no
    fallback path)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _call(name: str, *args) -> None:
    rc = getattr(lib(), name)(*args)
    if rc != MOE_OK:
        raise MoeError(name, rc, lib().moe_last_error().decode(errors="replace"))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _out(out: Optional[torch.Tensor], shape, dtype, like: torch.Tensor, name: str) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name}: out shape {tuple(out.shape)} != {tuple(shape)}")
    return out


def num_blocks(numel: int, E: int, block_m: int, padding_m: int) -> int:
    n = lib().moe_num_blocks(numel, E, block_m, padding_m)
    if n < 0:
        raise ValueError("num_blocks: padding_m must be a positive multiple of block_m")
    return int(n)


def align_workspace_bytes(numel: int, E: int) -> int:
    return int(lib().moe_align_workspace_bytes(numel, E))


# ----------------------------------------------------------------- entries --

def moe_topk_softmax(logits: torch.Tensor, top_k: int, topk_ids=None, topk_weights=None,
                     expert_bias: Optional[torch.Tensor] = None, scoring: str = "softmax",
                     renormalize: bool = True):
    T, E = logits.shape
    if scoring not in SCORING:
        raise ValueError(f"moe_topk_softmax: scoring must be one of {sorted(SCORING)}")
    ids = _out(topk_ids, (T, top_k), torch.int32, logits, "topk_ids")
    w = _out(topk_weights, (T, top_k), torch.float32, logits, "topk_weights")
    bias = None
    if expert_bias is not None:
        if tuple(expert_bias.shape) != (E,):
            raise ValueError("moe_topk_softmax: expert_bias must be [E]")
        bias = _ptr(expert_bias, torch.float32, "expert_bias")
    _call("moe_topk_softmax", _ptr(logits, torch.float32, "logits"), bias, T, E, top_k, SCORING[scoring],
          int(bool(renormalize)), _ptr(ids, torch.int32, "topk_ids"), _ptr(w, torch.float32, "topk_weights"),
          _stream(logits))
    return ids, w


def alloc_tables(numel: int, E: int, padding_m: int, block_m: int, device) -> Dict[str, torch.Tensor]:
    mb = num_blocks(numel, E, block_m, padding_m)
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "group_sizes": torch.empty(E, **i32), "group_offsets": torch.empty(E, **i32),
        "group_padded_offsets": torch.empty(E, **i32), "group_idx_for_bx": torch.empty(mb, **i32),
        "sorted_pair": torch.empty(numel, **i32), "pair_to_row": torch.empty(numel, **i32),
        "workspace": torch.empty(max(1, align_workspace_bytes(numel, E)), dtype=torch.uint8, device=device),
    }


def moe_align(topk_ids: torch.Tensor, E: int, padding_m: int, block_m: int,
              tables: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    T, k = topk_ids.shape
    tb = tables if tables is not None else alloc_tables(T * k, E, padding_m, block_m, topk_ids.device)
    i32 = torch.int32
    ws = tb["workspace"]
    _call("moe_align", _ptr(topk_ids, i32, "topk_ids"), T, k, E, padding_m, block_m,
          _ptr(tb["group_sizes"], i32, "group_sizes"), _ptr(tb["group_offsets"], i32, "group_offsets"),
          _ptr(tb["group_padded_offsets"], i32, "group_padded_offsets"),
          _ptr(tb["group_idx_for_bx"], i32, "group_idx_for_bx"), _ptr(tb["sorted_pair"], i32, "sorted_pair"),
          _ptr(tb["pair_to_row"], i32, "pair_to_row"), ws.data_ptr(), ws.numel(), _stream(topk_ids))
    return tb


def moe_align_noalloc(topk_ids: torch.Tensor, E: int, padding_m: int, block_m: int,
                      tables: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """moe_align without a workspace: the library's static per-device scratch
    holds the chunk histogram (calls that overlap on one GPU race; pair counts
    whose histogram exceeds moe_align_noalloc_max_scratch_bytes() are refused).
    With `tables` given, nothing is allocated."""
    T, k = topk_ids.shape
    tb = tables if tables is not None else alloc_tables(T * k, E, padding_m, block_m, topk_ids.device)
    i32 = torch.int32
    _call("moe_align_noalloc", _ptr(topk_ids, i32, "topk_ids"), T, k, E, padding_m, block_m,
          _ptr(tb["group_sizes"], i32, "group_sizes"), _ptr(tb["group_offsets"], i32, "group_offsets"),
          _ptr(tb["group_padded_offsets"], i32, "group_padded_offsets"),
          _ptr(tb["group_idx_for_bx"], i32, "group_idx_for_bx"), _ptr(tb["sorted_pair"], i32, "sorted_pair"),
          _ptr(tb["pair_to_row"], i32, "pair_to_row"), _stream(topk_ids))
    return tb


def moe_align_noalloc_max_scratch_bytes() -> int:
    return int(lib().moe_align_noalloc_max_scratch_bytes())


def moe_permute(hidden: torch.Tensor, sorted_pair: Optional[torch.Tensor], top_k: int, out=None,
                pair_to_row: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, H = hidden.shape
    x = _out(out, (T * top_k, H), torch.bfloat16, hidden, "x_perm")
    _call("moe_permute", _ptr(hidden, torch.bfloat16, "hidden"), _ptr(sorted_pair, torch.int32, "sorted_pair"),
          _ptr(pair_to_row, torch.int32, "pair_to_row"), T, top_k, H, _ptr(x, torch.bfloat16, "x_perm"),
          _stream(hidden))
    return x


def _table_ptrs(tables):
    if tables is None:
        return None, None, None, None
    i32 = torch.int32
    return (_ptr(tables["group_sizes"], i32, "group_sizes"), _ptr(tables["group_offsets"], i32, "group_offsets"),
            _ptr(tables["group_padded_offsets"], i32, "group_padded_offsets"),
            _ptr(tables["group_idx_for_bx"], i32, "group_idx_for_bx"))


def grouped_gemm_gate_up(x_perm: torch.Tensor, w_gate_up: torch.Tensor, tables: Optional[Dict[str, torch.Tensor]],
                         padding_m: int, block_m: int, fuse_swiglu: bool = True, out=None) -> torch.Tensor:
    """tables=None: dense single group (w_gate_up [2F, H] or [1, 2F, H])."""
    if w_gate_up.dim() == 2:
        w_gate_up = w_gate_up.unsqueeze(0)
    E, twoF, H = w_gate_up.shape
    F = twoF // 2
    numel = x_perm.shape[0]
    if x_perm.shape[1] != H:
        raise ValueError("grouped_gemm_gate_up: x_perm width != H")
    o = _out(out, (numel, F if fuse_swiglu else 2 * F), torch.bfloat16, x_perm, "out")
    _call("grouped_gemm_gate_up", _ptr(x_perm, torch.bfloat16, "x_perm"), _ptr(w_gate_up, torch.bfloat16, "w_gate_up"),
          *_table_ptrs(tables), numel, E, H, F, padding_m, block_m, int(bool(fuse_swiglu)),
          _ptr(o, torch.bfloat16, "out"), _stream(x_perm))
    return o


def grouped_gemm_gate_up_gather(hidden: torch.Tensor, w_gate_up: torch.Tensor, tables: Dict[str, torch.Tensor],
                                top_k: int, padding_m: int, block_m: int, fuse_swiglu: bool = True,
                                out=None) -> torch.Tensor:
    """grouped_gemm_gate_up on the permuted rows hidden[sorted_pair[r] // top_k]
    without writing them out (tables from moe_align, which must carry
    sorted_pair)."""
    if tables is None:
        raise ValueError("grouped_gemm_gate_up_gather: needs the dispatch tables")
    if w_gate_up.dim() == 2:
        w_gate_up = w_gate_up.unsqueeze(0)
    E, twoF, H = w_gate_up.shape
    F = twoF // 2
    T = hidden.shape[0]
    if hidden.shape[1] != H:
        raise ValueError("grouped_gemm_gate_up_gather: hidden width != H")
    numel = T * top_k
    sp = tables["sorted_pair"]
    if sp.numel() != numel:
        raise ValueError("grouped_gemm_gate_up_gather: sorted_pair length != T*top_k")
    o = _out(out, (numel, F if fuse_swiglu else 2 * F), torch.bfloat16, hidden, "out")
    _call("grouped_gemm_gate_up_gather", _ptr(hidden, torch.bfloat16, "hidden"), T, _ptr(sp, torch.int32, "sorted_pair"),
          top_k, _ptr(w_gate_up, torch.bfloat16, "w_gate_up"), *_table_ptrs(tables), numel, E, H, F, padding_m,
          block_m, int(bool(fuse_swiglu)), _ptr(o, torch.bfloat16, "out"), _stream(hidden))
    return o


def swiglu(gate_up: torch.Tensor, out=None) -> torch.Tensor:
    M, twoF = gate_up.shape
    h = _out(out, (M, twoF // 2), torch.bfloat16, gate_up, "h")
    _call("swiglu", _ptr(gate_up, torch.bfloat16, "gate_up"), M, twoF // 2, _ptr(h, torch.bfloat16, "h"),
          _stream(gate_up))
    return h


def grouped_gemm_down(h: torch.Tensor, w_down: torch.Tensor, tables: Optional[Dict[str, torch.Tensor]],
                      padding_m: int, block_m: int, out=None) -> torch.Tensor:
    if w_down.dim() == 2:
        w_down = w_down.unsqueeze(0)
    E, H, F = w_down.shape
    numel = h.shape[0]
    if h.shape[1] != F:
        raise ValueError("grouped_gemm_down: h width != F")
    y = _out(out, (numel, H), torch.bfloat16, h, "y")
    _call("grouped_gemm_down", _ptr(h, torch.bfloat16, "h"), _ptr(w_down, torch.bfloat16, "w_down"),
          *_table_ptrs(tables), numel, E, H, F, padding_m, block_m, _ptr(y, torch.bfloat16, "y"), _stream(h))
    return y


def moe_unpermute(y: torch.Tensor, pair_to_row: torch.Tensor, topk_weights: torch.Tensor,
                  routed_scaling_factor: float = 1.0, addend: Optional[torch.Tensor] = None,
                  out=None) -> torch.Tensor:
    T, k = topk_weights.shape
    H = y.shape[1]
    o = _out(out, (T, H), torch.bfloat16, y, "out")
    _call("moe_unpermute", _ptr(y, torch.bfloat16, "y"), _ptr(pair_to_row, torch.int32, "pair_to_row"),
          _ptr(topk_weights, torch.float32, "topk_weights"), T, k, H, float(routed_scaling_factor),
          _ptr(addend, torch.bfloat16, "addend"), _ptr(o, torch.bfloat16, "out"), _stream(y))
    return o


def swiglu_quant_fp8(gate_up: torch.Tensor, out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    M, twoF = gate_up.shape
    F = twoF // 2
    m_pad = -(-M // 128) * 128
    o = out or {}
    q_row = _out(o.get("q_row"), (M, F), torch.uint8, gate_up, "q_row")
    s_row = _out(o.get("s_row"), (M, F // 128), torch.float32, gate_up, "s_row")
    q_t = _out(o.get("q_t"), (F, m_pad), torch.uint8, gate_up, "q_t")
    s_t = _out(o.get("s_t"), (F // 128, m_pad // 128), torch.float32, gate_up, "s_t")
    _call("swiglu_quant_fp8", _ptr(gate_up, torch.bfloat16, "gate_up"), M, F, _ptr(q_row, torch.uint8, "q_row"),
          _ptr(s_row, torch.float32, "s_row"), _ptr(q_t, torch.uint8, "q_t"), _ptr(s_t, torch.float32, "s_t"),
          _stream(gate_up))
    return {"q_row": q_row, "s_row": s_row, "q_t": q_t, "s_t": s_t}


def tile_quant_fp8_m_pad_bound(M: int, E: int) -> int:
    return int(lib().tile_quant_fp8_m_pad_bound(M, E))


def tile_quant_fp8(x: torch.Tensor, group_sizes: Optional[torch.Tensor] = None, per_tile: bool = False,
                   swiglu: bool = False, m_pad: Optional[int] = None,
                   out: Optional[Dict[str, torch.Tensor]] = None, transposed: bool = True) -> Dict[str, torch.Tensor]:
    """Row (1x128) and grouped expand_128x transposed e4m3 quantization of x
    ([M, K] bf16, or gate_up [M, 2K] with swiglu=True). Without m_pad, q_t is
    ceil(M/128)*128 wide for one group and tile_quant_fp8_m_pad_bound(M, E)
    wide for E groups (the group sizes stay on the device). transposed=False:
    the row layout only ({"q_row", "s_row"})."""
    M, W = x.shape
    K = W // 2 if swiglu else W
    o = out or {}
    q_row = _out(o.get("q_row"), (M, K), torch.uint8, x, "q_row")
    s_row = _out(o.get("s_row"), (M, K // 128), torch.float32, x, "s_row")
    if not transposed:
        _call("tile_quant_fp8", _ptr(x, torch.bfloat16, "x"), M, K, int(swiglu), None, 0, 0, 0,
              _ptr(q_row, torch.uint8, "q_row"), _ptr(s_row, torch.float32, "s_row"), None, None, _stream(x))
        return {"q_row": q_row, "s_row": s_row}
    E = 0 if group_sizes is None else int(group_sizes.numel())
    if m_pad is None:
        m_pad = -(-M // 128) * 128 if group_sizes is None else tile_quant_fp8_m_pad_bound(M, E)
    q_t = _out(o.get("q_t"), (K, m_pad), torch.uint8, x, "q_t")
    s_t = _out(o.get("s_t"), ((K if per_tile else K // 128), m_pad // 128), torch.float32, x, "s_t")
    _call("tile_quant_fp8", _ptr(x, torch.bfloat16, "x"), M, K, int(swiglu), _ptr(group_sizes, torch.int32, "group_sizes"),
          E, int(per_tile), m_pad, _ptr(q_row, torch.uint8, "q_row"), _ptr(s_row, torch.float32, "s_row"),
          _ptr(q_t, torch.uint8, "q_t"), _ptr(s_t, torch.float32, "s_t"), _stream(x))
    return {"q_row": q_row, "s_row": s_row, "q_t": q_t, "s_t": s_t}


def fp8_block_quant_weights(w: torch.Tensor, out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """e4m3 codes of a bf16 weight [..., N, K] with one scale per 128x128 block: q like w (uint8), s [..., N/128, K/128]."""
    *lead, N, K = w.shape
    rows = int(np.prod(lead, dtype=np.int64)) * N if lead else N
    o = out or {}
    q = _out(o.get("q"), tuple(w.shape), torch.uint8, w, "q")
    s = _out(o.get("s"), (*lead, N // 128, K // 128), torch.float32, w, "s")
    _call("fp8_block_quant_weights", _ptr(w, torch.bfloat16, "w"), rows, K, _ptr(q, torch.uint8, "q"),
          _ptr(s, torch.float32, "s"), _stream(w))
    return {"q": q, "s": s}


def grouped_gemm_fp8(qa: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                     tables: Optional[Dict[str, torch.Tensor]], padding_m: int, block_m: int = 128,
                     out=None) -> torch.Tensor:
    if qw.dim() == 2:
        qw, sw = qw.unsqueeze(0), sw.unsqueeze(0)
    E, N, K = qw.shape
    numel = qa.shape[0]
    if qa.shape[1] != K:
        raise ValueError("grouped_gemm_fp8: qa width != K")
    y = _out(out, (numel, N), torch.bfloat16, qa, "y")
    _call("grouped_gemm_fp8", _ptr(qa, torch.uint8, "qa"), _ptr(sa, torch.float32, "sa"), _ptr(qw, torch.uint8, "qw"),
          _ptr(sw, torch.float32, "sw"), *_table_ptrs(tables), numel, E, N, K, padding_m, block_m,
          _ptr(y, torch.bfloat16, "y"), _stream(qa))
    return y


def grouped_gemm_gate_up_fp8(qa: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                             tables: Optional[Dict[str, torch.Tensor]], padding_m: int, block_m: int = 128,
                             fuse_swiglu: bool = True, top_k: Optional[int] = None, out=None) -> torch.Tensor:
    """Block-scaled FP8 gate_up: qa/sa the e4m3 codes and 1x128 scales of the
    compact permuted rows, or (top_k given) of the tokens, read through
    tables["sorted_pair"]; qw/sw = fp8_block_quant_weights(w_gate_up)."""
    if qw.dim() == 2:
        qw, sw = qw.unsqueeze(0), sw.unsqueeze(0)
    E, twoF, H = qw.shape
    F = twoF // 2
    a_rows = qa.shape[0]
    if qa.shape[1] != H:
        raise ValueError("grouped_gemm_gate_up_fp8: qa width != H")
    sp = None
    numel = a_rows
    if top_k is not None:
        if tables is None:
            raise ValueError("grouped_gemm_gate_up_fp8: the gather needs the dispatch tables")
        sp = tables["sorted_pair"]
        numel = a_rows * top_k
    o = _out(out, (numel, F if fuse_swiglu else 2 * F), torch.bfloat16, qa, "out")
    _call("grouped_gemm_gate_up_fp8", _ptr(qa, torch.uint8, "qa"), _ptr(sa, torch.float32, "sa"), a_rows,
          _ptr(sp, torch.int32, "sorted_pair"), int(top_k or 1), _ptr(qw, torch.uint8, "qw"),
          _ptr(sw, torch.float32, "sw"), *_table_ptrs(tables), numel, E, H, F, padding_m, block_m,
          int(bool(fuse_swiglu)), _ptr(o, torch.bfloat16, "out"), _stream(qa))
    return o
