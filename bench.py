#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config dsv3_prefill]

A step is one whole forward (routing, dispatch tables, permute, gate_up GEMM
with fused SwiGLU, down GEMM, shared expert, unpermute) over one batch of
seeded synthetic inputs that are resident in HBM before timing starts. The
SwiGLU + FP8 quantizer is timed on its own workload (M=32768, F=2048) in the
same run and reported under "kernels".

Prints one JSON line. `value` is forward TFLOP/s (6*T*k*H*F routed plus
6*T*H*Fs shared, per forward, over the timed steps); `ms_per_step` is ms per
forward. `roofline` is for the dominant kernel (grouped_gemm_gate_up): its
average duration comes from HIP events recorded on the launch stream around
every launch inside the timed region, which carries no other events (the
other stages' figures under "kernels" come from as many staged forwards, events
around every stage, after the timed region); the algorithmic bytes and FLOPs per
launch are counted from the realized routing (active experts' weights once,
activations in and out once). `cpu_baseline` times the oracle on a bounded
sample of tokens on the host cores. `other_workloads` times the same number
of whole forwards (`routed_moe_forward`, the shared expert on a second stream,
HIP events only around each forward) on the other forward shapes of the family
(the Qwen3 prefill and decode shapes, the Kimi-K2 table's token counts when
the DeepSeek-V3 prefill is the primary one), then as many replays of the same
forward captured as a HIP graph (`ms_per_forward_graph`), then as many staged
forwards (in line, events around every stage) for each one's per-kernel
figures.
`aligned_grouped_gemm` times the grouped GEMM alone on the aligned shapes of
the pages' grouped-GEMM baseline table (E groups of M rows each), with that
table's H200 figure beside each case as context. `grouped_quant` times the
grouped (expand_128x) FP8 quantizer on the pages' single-kernel benchmark
shapes; `fp8_down` the primary workload's down projection on the FP8 path
(1x128-tile e4m3 activations, 128x128-block e4m3 weights) beside the bf16 one,
and the whole forward with that FP8 down projection (`forward_ms`); then the
routed gate_up in FP8 (`gate_up_gemm_ms`) and the forward with both routed
GEMMs in FP8 (`forward_both_fp8_ms`), and with the shared expert's GEMMs in
FP8 as well (`forward_all_fp8_ms`).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="dsv3_prefill",
                   choices=["tiny", "qwen3_decode", "qwen3_prefill", "dsv3_prefill", "kimi_k2_t1", "kimi_k2_t32",
                            "kimi_k2_t512", "kimi_k2_t2048", "kimi_k2_t4096"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only-primary", action="store_true", help="skip the other forward workloads")
    p.add_argument("--fp8", action="store_true", help="with --only-primary: still run the FP8 leg (fp8_down)")
    p.add_argument("--gemm-table-only", action="store_true",
                   help="time only the aligned grouped-GEMM cases (prints their JSON object)")
    p.add_argument("--gemm-cases", default="all",
                   help="aligned grouped-GEMM cases to time: 'all', 'none' or a comma-separated list of names")
    p.add_argument("--cpu-tokens", type=int, default=4096, help="tokens in the oracle's timed sample (the whole T=4096 batch, about 11 s)")
    p.add_argument("--unfused", action="store_true", help="gate_up GEMM then a separate SwiGLU kernel")
    p.add_argument("--permute-copy", action="store_true",
                   help="permute as its own copy kernel instead of inside the gate_up GEMM's loads")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    return p.parse_args()


OTHER_WORKLOADS = ("qwen3_prefill", "qwen3_decode", "dsv3_prefill", "kimi_k2_t1", "kimi_k2_t32", "kimi_k2_t512",
                   "kimi_k2_t2048", "kimi_k2_t4096")
# context only (other hardware): the pages' H200 ms per forward of the Kimi-K2-scale
# routed + shared op (TileOPs #778 "Benchmark", TileOPs column) at each token count
KIMI_K2_PAGE_H200_MS = {1: 0.95, 32: 5.46, 512: 10.44, 2048: 19.99, 4096: 32.63}
STAGES = ("topk_softmax", "align", "permute", "gate_up", "swiglu", "down", "shared_gate_up", "shared_down",
          "unpermute")


class Workload:
    """One forward configuration: seeded inputs and weights resident on the GPU,
    the buffers of the forward, and a timed loop over whole forwards."""

    def __init__(self, cfg, dev, fuse, like=None, fuse_permute=True):
        import moe_synth
        import mixture_experts_routed_moe_amd as mx
        self.cfg, self.fuse, self.mx = cfg, fuse, mx
        self.hidden = moe_synth.hidden(cfg, dev)
        self.logits = moe_synth.router_logits(cfg, dev)
        self.bias = moe_synth.expert_bias(cfg, dev)
        if like is not None and like.cfg.cid == cfg.cid:
            # same workload id: the same weight tensors (only the token count differs)
            self.wgu, self.wd, self.swgu, self.swd = like.wgu, like.wd, like.swgu, like.swd
        else:
            self.wgu = moe_synth.w_gate_up(cfg, dev)
            self.wd = moe_synth.w_down(cfg, dev)
            self.swgu = moe_synth.shared_w_gate_up(cfg, dev) if cfg.shared_F else None
            self.swd = moe_synth.shared_w_down(cfg, dev) if cfg.shared_F else None
        shape = mx.MoEShape(cfg.T, cfg.H, cfg.F, cfg.E, cfg.top_k, cfg.padding_m, cfg.block_m, cfg.shared_F)
        self.bufs = mx.MoEBuffers(shape, dev, fuse_swiglu=fuse, fuse_permute=fuse_permute)

    def step(self, run):
        cfg, mx, bufs, fuse = self.cfg, self.mx, self.bufs, self.fuse
        tb = bufs.tables
        run("topk_softmax", lambda: mx.moe_topk_softmax(self.logits, cfg.top_k, bufs.topk_ids, bufs.topk_weights,
                                                        self.bias, cfg.scoring, cfg.renormalize))
        run("align", lambda: mx.moe_align(bufs.topk_ids, cfg.E, cfg.padding_m, cfg.block_m, tb))
        gu_out = bufs.h if fuse else bufs.gate_up
        if bufs.fuse_permute:
            # the permute folded into the gate_up GEMM's loads
            run("gate_up", lambda: mx.grouped_gemm_gate_up_gather(self.hidden, self.wgu, tb, cfg.top_k, cfg.padding_m,
                                                                  cfg.block_m, fuse, gu_out))
        else:
            run("permute", lambda: mx.moe_permute(self.hidden, tb["sorted_pair"], cfg.top_k, bufs.x_perm,
                                                  tb["pair_to_row"]))
            run("gate_up", lambda: mx.grouped_gemm_gate_up(bufs.x_perm, self.wgu, tb, cfg.padding_m, cfg.block_m,
                                                           fuse, gu_out))
        if not fuse:
            run("swiglu", lambda: mx.swiglu(bufs.gate_up, bufs.h))
        run("down", lambda: mx.grouped_gemm_down(bufs.h, self.wd, tb, cfg.padding_m, cfg.block_m, bufs.y))
        addend = None
        if cfg.shared_F:
            run("shared_gate_up", lambda: mx.grouped_gemm_gate_up(self.hidden, self.swgu, None, cfg.padding_m,
                                                                  cfg.block_m, True, bufs.shared_h))
            run("shared_down", lambda: mx.grouped_gemm_down(bufs.shared_h, self.swd, None, cfg.padding_m,
                                                            cfg.block_m, bufs.shared_y))
            addend = bufs.shared_y
        run("unpermute", lambda: mx.moe_unpermute(bufs.y, tb["pair_to_row"], bufs.topk_weights, cfg.rsf, addend,
                                                  bufs.out))

    def forward(self, side=None):
        """One forward through the library's composed forward (the shared
        expert on `side` when given)."""
        cfg = self.cfg
        return self.mx.routed_moe_forward(self.hidden, self.logits, self.wgu, self.wd, cfg.top_k, cfg.rsf,
                                          cfg.padding_m, cfg.block_m, self.swgu, self.swd, fuse_swiglu=self.fuse,
                                          buffers=self.bufs, expert_bias=self.bias, scoring=cfg.scoring,
                                          renormalize=cfg.renormalize, shared_stream=side,
                                          fuse_permute=self.bufs.fuse_permute)

    def run(self, steps, warmup, ev, whole=False, side=None, live=None):
        """Times `steps` forwards after `warmup` untimed ones. whole=False:
        each forward as its stages with HIP events around every stage (the
        per-kernel figures come from the timed region itself); with `live`
        (a stage name), events only around that stage's launch in the timed
        region, and the other stages' figures from as many staged forwards
        after it. whole=True: whole forwards through `routed_moe_forward`
        (shared expert on `side` when given) with events only around each
        forward, then the same number of staged forwards, in line, for the
        per-kernel figures."""
        import torch
        cfg, fuse = self.cfg, self.fuse
        ev_log = {s: [] for s in STAGES}

        def timed(name, fn):
            a = ev()
            fn()
            ev_log[name].append((a, ev()))

        for _ in range(warmup):
            if whole:
                self.forward(side)
            else:
                self.step(lambda name, fn: fn())
        torch.cuda.synchronize()
        print(f"# {cfg.name}: warmup done ({warmup} steps)", file=sys.stderr, flush=True)
        step_ev = []
        t0 = time.perf_counter()
        for _ in range(steps):
            a = ev()
            if whole:
                self.forward(side)
            elif live:
                self.step(lambda name, fn: timed(name, fn) if name == live else fn())
            else:
                self.step(timed)
            step_ev.append((a, ev()))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / steps
        print(f"# {cfg.name}: timed {steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
        graph_ms = None
        if whole:
            # the same forward captured once as a HIP graph, then replayed
            g = self.mx.MoEForwardGraph(self.hidden, self.logits, self.wgu, self.wd, cfg.top_k, cfg.rsf,
                                        cfg.padding_m, cfg.block_m, self.swgu, self.swd, fuse_swiglu=self.fuse,
                                        buffers=self.bufs, expert_bias=self.bias, scoring=cfg.scoring,
                                        renormalize=cfg.renormalize, shared_stream=side,
                                        fuse_permute=self.bufs.fuse_permute)
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            gev = []
            for _ in range(steps):
                a = ev()
                g.replay()
                gev.append((a, ev()))
            torch.cuda.synchronize()
            graph_ms = sum(a.elapsed_time(b) for a, b in gev) / len(gev)
            del g
        if whole or live:
            for _ in range(steps):
                self.step(lambda name, fn: fn() if name == live else timed(name, fn))
            torch.cuda.synchronize()

        stage_ms = {s: (sum(a.elapsed_time(b) for a, b in v) / len(v)) for s, v in ev_log.items() if v}
        stage_pct = {s: pct([a.elapsed_time(b) for a, b in v]) for s, v in ev_log.items() if v}
        step_pct = pct([a.elapsed_time(b) for a, b in step_ev])

        # realized routing (read after the timed region)
        gs = self.bufs.tables["group_sizes"].cpu().numpy()
        active = int((gs > 0).sum())
        numel, H, F, E = cfg.numel, cfg.H, cfg.F, cfg.E
        flop_gate_up = 4.0 * numel * H * F
        flop_down = 2.0 * numel * H * F
        flop_shared = 6.0 * cfg.T * H * cfg.shared_F
        flop_fwd = flop_gate_up + flop_down + flop_shared
        h_cols = F if fuse else 2 * F
        # algorithmic bytes (each pair's activation row counted once, numel*H*2,
        # as for a permuted copy); with the permute folded into the loads the
        # kernel's unique reads of the hidden states are T*H*2, reported beside
        bytes_gate_up = active * 2.0 * F * H * 2 + numel * H * 2 + numel * h_cols * 2
        bytes_gate_up_gathered = (active * 2.0 * F * H * 2 + (cfg.T if self.bufs.fuse_permute else numel) * H * 2
                                  + numel * h_cols * 2)
        bytes_down = active * 1.0 * H * F * 2 + numel * F * 2 + numel * H * 2
        bytes_permute = (cfg.T + numel) * H * 2 + 4 * numel
        bytes_unpermute = numel * H * 2 + 8 * cfg.T * cfg.top_k + cfg.T * H * 2 * (2 if cfg.shared_F else 1)

        def kern(name, flop, byts):
            ms = stage_ms.get(name)
            if not ms:
                return None
            s = ms * 1e-3
            return {"ms": round(ms, 4), **stage_pct[name], "tflops": round(flop / s / 1e12, 2) if flop else None,
                    "gbs": round(byts / s / 1e9, 1),
                    "mfma_frac": round(flop / s / 1e12 / BF16_PEAK_TFLOPS, 4) if flop else None,
                    "hbm_frac": round(byts / s / 1e9 / HBM_PEAK_GBS, 4),
                    "roofline_frac": round(max(flop / (BF16_PEAK_TFLOPS * 1e12), byts / (HBM_PEAK_GBS * 1e9)) / s, 4)}

        kernels = {
            "topk_softmax": kern("topk_softmax", 0, cfg.T * E * 4 + cfg.T * cfg.top_k * 8),
            "align": kern("align", 0, numel * 4 * 3),
            "permute": kern("permute", 0, bytes_permute),
            "grouped_gemm_gate_up": kern("gate_up", flop_gate_up, bytes_gate_up),
            "grouped_gemm_down": kern("down", flop_down, bytes_down),
            "unpermute": kern("unpermute", 0, bytes_unpermute),
        }
        if cfg.shared_F:
            Fs = cfg.shared_F
            kernels["shared_gate_up"] = kern("shared_gate_up", 4.0 * cfg.T * H * Fs,
                                             2.0 * Fs * H * 2 + cfg.T * H * 2 + cfg.T * Fs * 2)
            kernels["shared_down"] = kern("shared_down", 2.0 * cfg.T * H * Fs,
                                          1.0 * H * Fs * 2 + cfg.T * Fs * 2 + cfg.T * H * 2)
        gemm_s = (stage_ms["gate_up"] + stage_ms["down"]) * 1e-3
        summary = {
            "ms_per_forward": round(ms_per_step, 4), **{"step_" + k: v for k, v in step_pct.items()},
            "timing": ("whole forwards, shared expert on a second stream" if whole and side is not None and cfg.shared_F
                       else "whole forwards" if whole
                       else f"forwards with events around the {live} launch only (the other stages from as many "
                            "staged forwards after the timed region)" if live
                       else "staged forwards, events around every stage"),
            "ms_per_forward_graph": None if graph_ms is None else round(graph_ms, 4),
            "tflops_graph": None if graph_ms is None else round(flop_fwd / (graph_ms * 1e-3) / 1e12, 2),
            "tflops": round(flop_fwd / (ms_per_step * 1e-3) / 1e12, 2),
            "grouped_gemm_tflops": round((flop_gate_up + flop_down) / gemm_s / 1e12, 2),
            "grouped_gemm_mfma_frac": round((flop_gate_up + flop_down) / gemm_s / 1e12 / BF16_PEAK_TFLOPS, 4),
            "config": {"T": cfg.T, "H": H, "F": F, "E": E, "top_k": cfg.top_k, "padding_m": cfg.padding_m,
                       "shared_F": cfg.shared_F, "scoring": cfg.scoring, "active_experts": active,
                       "max_rows_per_expert": int(gs.max())},
            "kernels": kernels,
        }
        return {"ms_per_step": ms_per_step, "step_pct": step_pct, "stage_ms": stage_ms, "kernels": kernels,
                "flop_gate_up": flop_gate_up, "flop_down": flop_down, "flop_fwd": flop_fwd,
                "bytes_gate_up": bytes_gate_up, "bytes_gate_up_gathered": bytes_gate_up_gathered,
                "group_sizes": gs, "summary": summary}


def align_scaling(steps, warmup, ev, dev):
    """moe_align alone at growing pair counts (E = 256, top_k = 8, uniform
    random ids): its time should grow linearly with the pairs. The largest
    case, T = 262144 tokens, is the largest aligned-table token count."""
    import torch
    import mixture_experts_routed_moe_amd as mx
    out = {}
    for T in (4096, 32768, 262144):
        g = torch.Generator(device=dev).manual_seed(T)
        ids = torch.argsort(torch.rand(T, 256, device=dev, generator=g), dim=1)[:, :8].to(torch.int32).contiguous()
        tb = mx.alloc_tables(T * 8, 256, 128, 128, dev)
        for _ in range(warmup):
            mx.moe_align(ids, 256, 128, 128, tb)
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            a = ev()
            mx.moe_align(ids, 256, 128, 128, tb)
            evs.append((a, ev()))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in evs]
        out[f"T{T}_k8_E256"] = {"pairs": T * 8, "ms": round(sum(ms) / len(ms), 4), **pct(ms),
                                "ns_per_pair": round(sum(ms) / len(ms) * 1e6 / (T * 8), 3)}
        del ids, tb
    return out


def aligned_gemm_table(names, steps, warmup, ev, dev):
    """The grouped GEMM C[e] = A[e] @ B[e]^T on the aligned shapes of the pages'
    grouped-GEMM baseline table (E groups of exactly M rows), each timed with HIP
    events around every launch; the tables come from moe_align on a one-slot
    routing that sends M consecutive rows to each group, outside the timed loop."""
    import torch
    import moe_synth
    import mixture_experts_routed_moe_amd as mx
    out = {}
    for name in names:
        case = moe_synth.GEMM_CASES[name]
        T = case.E * case.M
        A = moe_synth.gemm_a(case, dev)
        W = moe_synth.gemm_w(case, dev)
        ids = torch.arange(case.E, dtype=torch.int32, device=dev).repeat_interleave(case.M).view(T, 1)
        tb = mx.moe_align(ids, case.E, 128, 128)
        y = torch.empty(T, case.N, dtype=torch.bfloat16, device=dev)
        for _ in range(warmup):
            mx.grouped_gemm_down(A, W, tb, 128, 128, y)
        evs = []
        for _ in range(steps):
            a = ev()
            mx.grouped_gemm_down(A, W, tb, 128, 128, y)
            evs.append((a, ev()))
        torch.cuda.synchronize()
        ms_list = [a.elapsed_time(b) for a, b in evs]
        ms = sum(ms_list) / len(ms_list)
        flop = 2.0 * T * case.N * case.K
        byts = 2.0 * (T * case.K + case.E * case.N * case.K + T * case.N)
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"M": case.M, "N": case.N, "K": case.K, "E": case.E, "ms": round(ms, 4), **pct(ms_list),
                     "tflops": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                     "roofline_frac": round(max(flop / (BF16_PEAK_TFLOPS * 1e12), byts / (HBM_PEAK_GBS * 1e9))
                                            / (ms * 1e-3), 4),
                     "page_h200_tflops": case.page_tflops}
        print(f"# aligned GEMM {name}: {ms:.3f} ms, {tf:.0f} TFLOP/s", file=sys.stderr, flush=True)
        del A, W, y, tb, ids
        torch.cuda.empty_cache()
    return out


def grouped_quant_table(steps, warmup, ev, dev):
    """The 1x128-tile FP8 quantizer with the grouped expand_128x transposed
    layout on the pages' single-kernel benchmark shapes (256 expert groups),
    per-block and per-tile transposed scales; HIP events around each launch,
    a 512 MiB read between launches."""
    import torch
    import moe_synth
    import mixture_experts_routed_moe_amd as mx
    out = {}
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    for name, per_tile in (("quant_131072x6144_e256", False), ("quant_131072x6144_e256", True),
                           ("swiglu_quant_131072x8192_e256", False)):
        case = moe_synth.GROUPED_QUANT_CASES[name]
        sizes = moe_synth.grouped_quant_sizes(case)
        x = moe_synth.grouped_quant_input(case, dev)
        gs = torch.as_tensor(sizes, device=dev)
        m_pad = int(((sizes + 127) // 128).sum() * 128)
        bufs = mx.tile_quant_fp8(x, gs, per_tile=per_tile, swiglu=case.swiglu, m_pad=m_pad)
        for _ in range(warmup):
            mx.tile_quant_fp8(x, gs, per_tile=per_tile, swiglu=case.swiglu, m_pad=m_pad, out=bufs)
        evs = []
        for _ in range(max(10, steps)):
            flush.sum()
            a = ev()
            mx.tile_quant_fp8(x, gs, per_tile=per_tile, swiglu=case.swiglu, m_pad=m_pad, out=bufs)
            evs.append((a, ev()))
        torch.cuda.synchronize()
        ms_list = [a.elapsed_time(b) for a, b in evs]
        ms = sum(ms_list) / len(ms_list)
        K, M = case.K, case.M
        byts = (M * K * 2 * (2 if case.swiglu else 1) + M * K + 4 * M * K // 128 + K * m_pad
                + 4 * (K if per_tile else K // 128) * (m_pad // 128))
        key = f"{name}_{'per_tile' if per_tile else 'per_block'}"
        out[key] = {"M": M, "K": K, "E": case.E, "swiglu": case.swiglu, "m_pad": m_pad, "ms": round(ms, 4),
                    **pct(ms_list), "gbs": round(byts / ms / 1e6, 1), "hbm_frac": round(byts / ms / 1e6 / HBM_PEAK_GBS, 4)}
        print(f"# grouped quant {key}: {ms * 1e3:.1f} us, {byts / ms / 1e6:.0f} GB/s", file=sys.stderr, flush=True)
        del x, bufs, gs
        torch.cuda.empty_cache()
    del flush
    return out


def fp8_down(wl, steps, warmup, ev):
    """The down projection on the FP8 path for the workload's routing: h (the
    forward's bf16 SwiGLU output, left in the buffers by the timed forwards)
    quantized to 1x128-tile e4m3 codes (tile_quant_fp8), then the
    block-scaled FP8 grouped GEMM against 128x128-block e4m3 weights prepared
    once. HIP events around each launch; FLOP as for the bf16 down."""
    import torch
    mx, cfg, bufs = wl.mx, wl.cfg, wl.bufs
    qw = mx.fp8_block_quant_weights(wl.wd)
    qa = mx.tile_quant_fp8(bufs.h, None)
    y = torch.empty_like(bufs.y)
    for _ in range(warmup):
        mx.tile_quant_fp8(bufs.h, None, out=qa)
        mx.grouped_gemm_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], bufs.tables, cfg.padding_m, cfg.block_m, y)
    eq, eg = [], []
    for _ in range(steps):
        a = ev()
        mx.tile_quant_fp8(bufs.h, None, out=qa)
        b = ev()
        mx.grouped_gemm_fp8(qa["q_row"], qa["s_row"], qw["q"], qw["s"], bufs.tables, cfg.padding_m, cfg.block_m, y)
        eg.append((b, ev()))
        eq.append((a, b))
    torch.cuda.synchronize()
    q_ms = sum(a.elapsed_time(b) for a, b in eq) / len(eq)
    g_list = [a.elapsed_time(b) for a, b in eg]
    g_ms = sum(g_list) / len(g_list)
    flop = 2.0 * cfg.numel * cfg.H * cfg.F
    # whole forwards with the routed down projection in FP8 (row-layout codes of h)
    b8 = mx.MoEBuffers(wl.bufs.shape, wl.hidden.device, wl.fuse, wl.bufs.fuse_permute, fp8_down=True)

    def fwd8():
        mx.routed_moe_forward(wl.hidden, wl.logits, wl.wgu, wl.wd, cfg.top_k, cfg.rsf, cfg.padding_m, cfg.block_m,
                              wl.swgu, wl.swd, fuse_swiglu=wl.fuse, buffers=b8, expert_bias=wl.bias,
                              scoring=cfg.scoring, renormalize=cfg.renormalize, fuse_permute=wl.bufs.fuse_permute,
                              w_down_fp8=qw)
    for _ in range(warmup):
        fwd8()
    ef = []
    for _ in range(steps):
        a = ev()
        fwd8()
        ef.append((a, ev()))
    torch.cuda.synchronize()
    f_ms = sum(a.elapsed_time(b) for a, b in ef) / len(ef)
    flop_fwd = 6.0 * cfg.numel * cfg.H * cfg.F + 6.0 * cfg.T * cfg.H * cfg.shared_F
    del b8
    # the routed gate_up in FP8 too: the GEMM alone (codes of the hidden states
    # read through the permutation), then whole forwards with both FP8 GEMMs
    qg = mx.fp8_block_quant_weights(wl.wgu)
    qh = mx.tile_quant_fp8(wl.hidden, transposed=False)
    hg = torch.empty_like(bufs.h)
    for _ in range(warmup):
        mx.grouped_gemm_gate_up_fp8(qh["q_row"], qh["s_row"], qg["q"], qg["s"], bufs.tables, cfg.padding_m,
                                    top_k=cfg.top_k, out=hg)
    eu = []
    for _ in range(steps):
        a = ev()
        mx.grouped_gemm_gate_up_fp8(qh["q_row"], qh["s_row"], qg["q"], qg["s"], bufs.tables, cfg.padding_m,
                                    top_k=cfg.top_k, out=hg)
        eu.append((a, ev()))
    torch.cuda.synchronize()
    u_ms = sum(a.elapsed_time(b) for a, b in eu) / len(eu)
    b88 = mx.MoEBuffers(wl.bufs.shape, wl.hidden.device, wl.fuse, True, fp8_down=True, fp8_gate_up=True)

    def fwd88():
        mx.routed_moe_forward(wl.hidden, wl.logits, wl.wgu, wl.wd, cfg.top_k, cfg.rsf, cfg.padding_m, cfg.block_m,
                              wl.swgu, wl.swd, fuse_swiglu=wl.fuse, buffers=b88, expert_bias=wl.bias,
                              scoring=cfg.scoring, renormalize=cfg.renormalize, w_down_fp8=qw, w_gate_up_fp8=qg)
    for _ in range(warmup):
        fwd88()
    e88 = []
    for _ in range(steps):
        a = ev()
        fwd88()
        e88.append((a, ev()))
    torch.cuda.synchronize()
    f88_ms = sum(a.elapsed_time(b) for a, b in e88) / len(e88)
    del b88, hg
    # and the shared expert's GEMMs in FP8 as well
    f4_ms = None
    if cfg.shared_F:
        qs = {"gate_up": mx.fp8_block_quant_weights(wl.swgu), "down": mx.fp8_block_quant_weights(wl.swd)}
        b4 = mx.MoEBuffers(wl.bufs.shape, wl.hidden.device, wl.fuse, True, fp8_down=True, fp8_gate_up=True,
                           fp8_shared=True)

        def fwd4():
            mx.routed_moe_forward(wl.hidden, wl.logits, wl.wgu, wl.wd, cfg.top_k, cfg.rsf, cfg.padding_m,
                                  cfg.block_m, wl.swgu, wl.swd, fuse_swiglu=wl.fuse, buffers=b4, expert_bias=wl.bias,
                                  scoring=cfg.scoring, renormalize=cfg.renormalize, w_down_fp8=qw, w_gate_up_fp8=qg,
                                  w_shared_fp8=qs)
        for _ in range(warmup):
            fwd4()
        e4 = []
        for _ in range(steps):
            a = ev()
            fwd4()
            e4.append((a, ev()))
        torch.cuda.synchronize()
        f4_ms = sum(a.elapsed_time(b) for a, b in e4) / len(e4)
        del b4, qs
    del qg
    flop_gu = 4.0 * cfg.numel * cfg.H * cfg.F
    return {"gemm_ms": round(g_ms, 4), **pct(g_list), "quant_h_ms": round(q_ms, 4),
            "forward_ms": round(f_ms, 4), "forward_tflops": round(flop_fwd / (f_ms * 1e-3) / 1e12, 2),
            "gate_up_gemm_ms": round(u_ms, 4), "gate_up_tflops": round(flop_gu / (u_ms * 1e-3) / 1e12, 2),
            "forward_both_fp8_ms": round(f88_ms, 4),
            "forward_both_fp8_tflops": round(flop_fwd / (f88_ms * 1e-3) / 1e12, 2),
            "forward_all_fp8_ms": None if f4_ms is None else round(f4_ms, 4),
            "forward_all_fp8_tflops": None if f4_ms is None else round(flop_fwd / (f4_ms * 1e-3) / 1e12, 2),
            "tflops": round(flop / (g_ms * 1e-3) / 1e12, 2),
            "fp8_mfma_frac": round(flop / (g_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
            "bf16_mfma_frac": round(flop / (g_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the multi-GPU (expert-parallel / tensor-parallel) path is "
              "not built, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_synth
    import mixture_experts_routed_moe_amd as mx

    dev = torch.device("cuda", 0)
    cfg = moe_synth.CONFIGS[args.config]
    fuse = not args.unfused
    if args.gemm_table_only:
        stream0 = torch.cuda.current_stream(dev)

        def ev0():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream0)
            return e
        names = list(moe_synth.GEMM_CASES) if args.gemm_cases in ("all", "none") else args.gemm_cases.split(",")
        print(json.dumps({"aligned_grouped_gemm": aligned_gemm_table(names, args.steps, args.warmup, ev0, dev)}),
              flush=True)
        return
    t_gen = time.time()
    wl = Workload(cfg, dev, fuse, fuse_permute=not args.permute_copy)
    qx = moe_synth.quant_input(moe_synth.QUANT_CONFIG.M, moe_synth.QUANT_CONFIG.F, dev)
    qbufs = mx.swiglu_quant_fp8(qx)
    torch.cuda.synchronize()
    print(f"# inputs generated on the GPU in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    res = wl.run(args.steps, args.warmup, ev, live="gate_up")
    ms_per_step = res["ms_per_step"]
    stage_ms, kernels = res["stage_ms"], res["kernels"]
    flop_gate_up, bytes_gate_up, flop_down = res["flop_gate_up"], res["bytes_gate_up"], res["flop_down"]
    gs = res["group_sizes"]
    active = int((gs > 0).sum())
    H, F, E = cfg.H, cfg.F, cfg.E
    hidden, logits, bias, wgu, wd, swgu, swd = (wl.hidden, wl.logits, wl.bias, wl.wgu, wl.wd, wl.swgu, wl.swd)

    fp8 = None if args.only_primary and not args.fp8 else fp8_down(wl, args.steps, args.warmup, ev)
    if fp8 is not None:
        fp8["bf16_down_ms"] = round(stage_ms["down"], 4)
        print(f"# fp8 down: {fp8['gemm_ms']:.3f} ms (bf16 {stage_ms['down']:.3f} ms)", file=sys.stderr, flush=True)

    # the other forward workloads of the same family: whole forwards, the
    # shared expert (where there is one) on a second stream of default priority
    others = {}
    side = torch.cuda.Stream(dev)
    for name in OTHER_WORKLOADS:
        if name == cfg.name or args.only_primary:
            continue
        prev = wl
        del wl
        if prev.cfg.cid != moe_synth.CONFIGS[name].cid:
            prev = None
            torch.cuda.empty_cache()
        wl = Workload(moe_synth.CONFIGS[name], dev, fuse, like=prev, fuse_permute=not args.permute_copy)
        del prev
        r = wl.run(args.steps, args.warmup, ev, whole=True, side=side)
        others[name] = r["summary"]
        if name.startswith("kimi_k2_t"):
            others[name]["page_h200_ms"] = KIMI_K2_PAGE_H200_MS.get(moe_synth.CONFIGS[name].T)
        print(f"# {name}: {r['ms_per_step']:.3f} ms/forward", file=sys.stderr, flush=True)

    # aligned grouped GEMM at the pages' table shapes
    if args.gemm_cases == "none":
        gemm_names = []
    elif args.gemm_cases == "all":
        gemm_names = list(moe_synth.GEMM_CASES)
    else:
        gemm_names = args.gemm_cases.split(",")
    gemm_table = aligned_gemm_table(gemm_names, args.steps, args.warmup, ev, dev) if gemm_names else {}

    grouped_quant = {} if args.only_primary else grouped_quant_table(args.steps, args.warmup, ev, dev)
    align = {} if args.only_primary else align_scaling(args.steps, args.warmup, ev, dev)

    # fused SwiGLU + FP8 quantizer on its own workload, HIP events around each launch
    qM, qF = moe_synth.QUANT_CONFIG.M, moe_synth.QUANT_CONFIG.F
    for _ in range(5):
        mx.swiglu_quant_fp8(qx, qbufs)
    # its working set (about 0.4 GB) is under twice the 256 MiB MALL: reading a
    # 512 MiB buffer outside the events evicts it between launches (a read, so
    # the timed launch does not also pay for writing dirty flush lines back)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    qev = []
    for i in range(max(20, args.steps)):
        flush.sum()
        a = ev()
        mx.swiglu_quant_fp8(qx, qbufs)
        qev.append((a, ev()))
    torch.cuda.synchronize()
    del flush
    q_list = [a.elapsed_time(b) for a, b in qev]
    q_ms = sum(q_list) / len(q_list)
    qm_pad = -(-qM // 128) * 128
    q_bytes = qM * 4 * qF + qM * qF + 4 * qM * qF // 128 + qF * qm_pad + 4 * (qF // 128) * (qm_pad // 128)
    kernels["swiglu_quant_fp8"] = {"workload": f"M={qM},F={qF}", "ms": round(q_ms, 4), **pct(q_list),
                                   "mall_flushed": True,
                                   "gbs": round(q_bytes / q_ms / 1e6, 1),
                                   "hbm_frac": round(q_bytes / q_ms / 1e6 / HBM_PEAK_GBS, 4)}

    if args.copy_calibration:
        # a plain streaming kernel of known size: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    gu = kernels["grouped_gemm_gate_up"]
    gu_s = stage_ms["gate_up"] * 1e-3
    roofline = {"kernel": "grouped_gemm_gate_up" + ("(+swiglu)" if fuse else ""),
                "bound": "hbm" if bytes_gate_up / (HBM_PEAK_GBS * 1e9) >= flop_gate_up / (BF16_PEAK_TFLOPS * 1e12) else "mfma",
                "achieved": None, "peak": None, "unit": None, "frac": None, "traffic": None,
                "bytes_per_launch": bytes_gate_up, "flop_per_launch": flop_gate_up,
                "bytes_convention": "active experts' weights + numel*H*2 activations in + numel*F*2 out",
                "bytes_per_launch_gathered": res["bytes_gate_up_gathered"],
                "frac_gathered": round(res["bytes_gate_up_gathered"] / gu_s / 1e9 / HBM_PEAK_GBS, 4),
                "launch_ms": round(stage_ms["gate_up"], 4), "mfma_frac": gu["mfma_frac"], "hbm_frac": gu["hbm_frac"]}
    if roofline["bound"] == "hbm":
        roofline.update(achieved=round(bytes_gate_up / gu_s / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        roofline.update(achieved=round(flop_gate_up / gu_s / 1e12, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s")
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)
    roofline["traffic"] = measured_traffic(cfg.name, fuse)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, hidden, logits, bias, wgu, wd, swgu, swd, args.cpu_tokens)

    step_pct, flop_fwd = res["step_pct"], res["flop_fwd"]
    value = flop_fwd / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": "routed-experts fwd ms + grouped-GEMM TFLOPS (% MFMA peak), T=4096",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "step_ms_p50": step_pct["ms_p50"], "step_ms_min": step_pct["ms_min"],
        "step_ms_p90": step_pct["ms_p90"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "timing": res["summary"]["timing"], "dtype": "bf16", "data": "synthetic (router logits N(0,1) from numpy PCG64; hidden states and random-init weights from a seeded counter-based generator)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": H, "F": F, "E": E, "top_k": cfg.top_k,
                   "padding_m": cfg.padding_m, "block_m": cfg.block_m, "routed_scaling_factor": cfg.rsf,
                   "zipf_bias_s": cfg.zipf_s, "shared_F": cfg.shared_F, "fused_swiglu": fuse, "fused_permute": not args.permute_copy,
                   "active_experts": active, "max_rows_per_expert": int(gs.max()),
                   "parallelism": "single GPU"},
        "grouped_gemm_tflops": round((flop_gate_up + flop_down) / ((stage_ms["gate_up"] + stage_ms["down"]) * 1e-3) / 1e12, 2),
        "grouped_gemm_mfma_frac": round((flop_gate_up + flop_down) / ((stage_ms["gate_up"] + stage_ms["down"]) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "other_workloads": others,
        "aligned_grouped_gemm": gemm_table,
        "grouped_quant": grouped_quant,
        "align_scaling": align,
        "fp8_down": fp8,
    }
    print(json.dumps(line), flush=True)


def gemm_source_sha() -> str:
    """First 16 hex digits of the sha256 over the GEMM kernels' code (gemm.hip,
    then wide_sched.h, then moe_common.h, each with its // comments, trailing
    blanks and empty lines removed; the files hold no // inside a string and
    no block comment): the revision a traffic figure belongs to, unchanged by
    an edit of comments only."""
    import hashlib
    h = hashlib.sha256()
    for name in ("gemm.hip", "wide_sched.h", "moe_common.h"):
        with open(os.path.join(ROOT, "mixture_experts_routed_moe_amd", "csrc", name), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload, fused):
    """HBM bytes per launch of the routed gate_up GEMM from the committed rocprofv3
    FETCH_SIZE + WRITE_SIZE summary (scaled by the copy calibration), or None when
    that summary is for another workload or another revision of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"grouped_gemm_gate_up_{workload}.txt")
    if not fused or not os.path.exists(path):
        return None
    kv = dict(line.split("=", 1) for line in open(path).read().splitlines() if "=" in line and not line.startswith("#"))
    sha = gemm_source_sha()
    if kv.get("kernel_source_sha256_16") != sha:
        return None
    return int(float(kv["traffic_bytes"]))


def pct(ms_list):
    v = np.sort(np.asarray(ms_list, dtype=np.float64))
    return {"ms_p50": round(float(np.percentile(v, 50)), 4), "ms_min": round(float(v[0]), 4),
            "ms_p90": round(float(np.percentile(v, 90)), 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, hidden, logits, bias, wgu, wd, swgu, swd, n_tokens):
    """The oracle, as it stands, on a bounded sample of tokens: TFLOP/s on the host cores."""
    import torch
    import moe_synth
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(1234)
    tokens = np.sort(rng.choice(cfg.T, size=min(n_tokens, cfg.T), replace=False))
    tsel = torch.as_tensor(tokens, device=hidden.device)
    hid = moe_synth.bits16(hidden[tsel])
    lg = logits[tsel].cpu().numpy()
    bias_h = None if bias is None else bias.cpu().numpy()
    ids, _ = oracle.route(lg, cfg.top_k, bias_h, cfg.scoring, cfg.renormalize)
    used = np.unique(ids)
    sel = torch.as_tensor(used, device=wgu.device)
    wgu_h = moe_synth.bits16(wgu[sel])
    wd_h = moe_synth.bits16(wd[sel])
    swgu_h = moe_synth.bits16(swgu) if swgu is not None else None
    swd_h = moe_synth.bits16(swd) if swd is not None else None
    remap = np.zeros(cfg.E, np.int64)
    remap[used] = np.arange(used.size)
    # the oracle's forward on the sampled tokens, restricted to the experts they reach
    t0 = time.perf_counter()
    ids2, w = oracle.route(lg, cfg.top_k, bias_h, cfg.scoring, cfg.renormalize)
    ids_r = remap[ids2].astype(np.int32)
    tab = oracle.dispatch_tables(ids_r, used.size, cfg.padding_m, cfg.block_m)
    xp = oracle.permute(hid, tab["sorted_pair"], cfg.top_k)
    gu = oracle.grouped_gemm(xp, wgu_h, tab["group_sizes"], tab["group_offsets"])
    h = oracle.swiglu(gu, cfg.F)
    y = oracle.grouped_gemm(h, wd_h, tab["group_sizes"], tab["group_offsets"])
    shared = oracle.shared_expert(hid, swgu_h, swd_h) if swgu_h is not None else None
    oracle.unpermute(y, tab["pair_to_row"], w, cfg.top_k, cfg.rsf, shared)
    dt = time.perf_counter() - t0
    flop = 6.0 * tokens.size * cfg.top_k * cfg.H * cfg.F + 6.0 * tokens.size * cfg.H * cfg.shared_F
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{tokens.size} of {cfg.T} tokens of {cfg.name} ({used.size} experts reached), "
                      f"full forward incl. shared expert, float64 GEMMs; {dt:.1f}s",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
