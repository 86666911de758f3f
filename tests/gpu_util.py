"""Helpers shared by the GPU parity tests (host side only)."""
import sys

import numpy as np
import torch

import moe_synth
import oracle
from oracle import numerics as nm

BF16_ATOL = 1e-2
BF16_RTOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda", 0)


def bits(t: torch.Tensor) -> np.ndarray:
    return moe_synth.bits16(t)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_bf16_close(got_bits: np.ndarray, ref_bits: np.ndarray, name: str,
                      atol: float = BF16_ATOL, rtol: float = BF16_RTOL):
    g = nm.bf16_to_f64(got_bits)
    r = nm.bf16_to_f64(ref_bits)
    assert g.shape == r.shape, f"{name}: shape {g.shape} != {r.shape}"
    bad = np.abs(g - r) > atol + rtol * np.abs(r)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside atol={atol} rtol={rtol}; "
                             f"first {idx.tolist()}: got {g[bad][:5]} ref {r[bad][:5]}")
    return float(np.abs(g - r).max()) if g.size else 0.0


def inputs(cfg, device):
    d = {
        "hidden": moe_synth.hidden(cfg, device),
        "logits": moe_synth.router_logits(cfg, device),
        "w_gate_up": moe_synth.w_gate_up(cfg, device),
        "w_down": moe_synth.w_down(cfg, device),
    }
    if cfg.zipf_s is not None:
        d["bias"] = moe_synth.expert_bias(cfg, device)
    if cfg.shared_F:
        d["shared_w_gate_up"] = moe_synth.shared_w_gate_up(cfg, device)
        d["shared_w_down"] = moe_synth.shared_w_down(cfg, device)
    return d


def oracle_tokens(cfg, inp, tokens):
    """Oracle outputs for a subset of tokens (each token's output depends only on its row).

    Routing uses the tokens' full logit rows; the experts they reach are
    gathered (weights copied from the generator's device tensors) and the
    oracle's stages run on that subset.
    """
    tokens = np.asarray(tokens)
    hid = bits(inp["hidden"][torch.as_tensor(tokens, device=inp["hidden"].device)])
    logits = host(inp["logits"][torch.as_tensor(tokens, device=inp["logits"].device)])
    ids, w = oracle.route(logits, cfg.top_k, host(inp["bias"]) if "bias" in inp else None, cfg.scoring,
                          cfg.renormalize)
    used = np.unique(ids)
    remap = {int(e): i for i, e in enumerate(used)}
    ids_r = np.vectorize(lambda e: remap[int(e)])(ids).astype(np.int32)
    sel = torch.as_tensor(used, device=inp["w_gate_up"].device)
    wgu = bits(inp["w_gate_up"][sel])
    wd = bits(inp["w_down"][sel])
    tab = oracle.dispatch_tables(ids_r, len(used), cfg.padding_m, cfg.block_m)
    xp = oracle.permute(hid, tab["sorted_pair"], cfg.top_k)
    gu = oracle.grouped_gemm(xp, wgu, tab["group_sizes"], tab["group_offsets"])
    h = oracle.swiglu(gu, cfg.F)
    y = oracle.grouped_gemm(h, wd, tab["group_sizes"], tab["group_offsets"])
    shared = None
    if cfg.shared_F:
        shared = oracle.shared_expert(hid, bits(inp["shared_w_gate_up"]), bits(inp["shared_w_down"]))
    out = oracle.unpermute(y, tab["pair_to_row"], w, cfg.top_k, cfg.rsf, shared)
    routed = oracle.unpermute(y, tab["pair_to_row"], w, cfg.top_k, cfg.rsf, None)
    return {"topk_ids": ids, "topk_weights": w, "out": out, "shared": shared, "routed": routed, "gate_up": gu,
            "h": h, "y": y, "tables": tab, "w_down_used": wd}


def bf16_ulp(bits_arr: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at each element (2^(e-7) in binade [2^e, 2^(e+1)), 2^-133 below 2^-126)."""
    v = np.abs(nm.bf16_to_f64(bits_arr))
    _, e = np.frexp(v)
    return np.ldexp(1.0, np.maximum(e - 8, -133))
