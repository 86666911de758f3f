"""Seeded synthetic inputs for the routed-expert MoE forward and the fused
SwiGLU + FP8 quantizer.

This module holds the workload shapes and the random inputs only. It performs
no step of the method (no routing, no tables, no GEMM, no activation, no
quantization), so the oracle and the HIP path can both take their inputs from
here without sharing any of the method's arithmetic.

Generator
---------
Every element is a pure function of (tensor key, element index): a 32-bit
integer hash ("lowbias32", an xorshift-multiply mixer published by C. Wellons
in the hash-prospector project) feeds four 22-bit uniform integers whose sum
is an Irwin-Hall(4) variate. Centred and scaled, it approximates N(0, sigma^2)
with mean 0, the requested variance and tails cut at +-3.46 sigma:

    S = u1 + u2 + u3 + u4          (integer, exact)
    z = float32(S - 2*(2^22-1)) * float32(sigma / sqrt(4*(2^44-1)/12))

S - mean is below 2^24 in magnitude, so the conversion is exact and the single
float32 multiply is correctly rounded on any IEEE device. bf16 tensors are
that float32 value rounded to nearest-even by torch. The arithmetic is written
in torch int64 ops, so CPU and GPU produce the same bits, and any index range
of a tensor (one expert's weights, one token's row) can be regenerated alone.

The router logits are the exception: they are drawn from a true normal on the
host (see router_logits), because the tails decide which experts a biased
routing reaches.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

_M32 = 0xFFFFFFFF
_U22 = (1 << 22) - 1
_IH_MEAN = 2 * _U22                     # mean of the sum of four uniforms on [0, 2^22-1]
_IH_STD = math.sqrt(4.0 * ((_U22 + 1) ** 2 - 1) / 12.0)


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for 0 <= x < 2^32, kept inside int64 without overflow."""
    lo = c & 0xFFFF
    hi = c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 integer mixer on values in [0, 2^32)."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def tensor_key(*parts: int) -> int:
    """32-bit key for a tensor from small integers (workload id, tensor tag, ...)."""
    k = 0x6A09E667
    for p in parts:
        k = _mix32_int(k ^ _mix32_int(int(p) + 0x9E3779B9))
    return k


def _normal_f32_range(key: int, start: int, stop: int, sigma: float,
                      device: torch.device | str) -> torch.Tensor:
    n = stop - start
    if n <= 0:
        return torch.empty(0, dtype=torch.float32, device=device)
    i = torch.arange(start, stop, dtype=torch.int64, device=device)
    base = _mix32(_mix32((i & _M32) ^ key) ^ ((i >> 32) & _M32))
    h1 = _mix32(base ^ 0x85EBCA6B)
    h2 = _mix32(base ^ 0xC2B2AE35)
    h3 = _mix32(base ^ 0x27D4EB2F)
    del base, i
    u4 = ((h1 >> 22) | ((h2 >> 22) << 10) | ((h3 >> 22) << 20)) & _U22
    s = (h1 & _U22) + (h2 & _U22) + (h3 & _U22) + u4
    del h1, h2, h3, u4
    z = (s - _IH_MEAN).to(torch.float32)
    scale = torch.tensor(sigma / _IH_STD, dtype=torch.float32)
    return z * scale.to(device)


def normal_f32(key: int, shape: Sequence[int], sigma: float = 1.0,
               device: torch.device | str = "cpu", start: int = 0,
               chunk: int = 1 << 26) -> torch.Tensor:
    """float32 tensor of `shape` holding elements start.. of the keyed stream."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=torch.float32, device=device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        out[c0:c1] = _normal_f32_range(key, start + c0, start + c1, sigma, device)
    return out.view(*shape)


def normal_bf16(key: int, shape: Sequence[int], sigma: float = 1.0,
                device: torch.device | str = "cpu", start: int = 0,
                chunk: int = 1 << 26) -> torch.Tensor:
    """bf16 tensor: the float32 stream rounded to nearest-even by torch."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        out[c0:c1] = _normal_f32_range(key, start + c0, start + c1, sigma, device).to(torch.bfloat16)
    return out.view(*shape)


def bits16(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 tensor as a host uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
TAG_HIDDEN, TAG_LOGITS, TAG_BIAS, TAG_WGU, TAG_WD, TAG_SWGU, TAG_SWD, TAG_QUANT = range(8)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One routed-expert forward workload.

    hidden [T,H] bf16 ~N(0,1); router logits [T,E] fp32 ~N(0,1), plus a per-expert
    Zipf bias [E] (expert_bias) when `zipf_s` is set; w_gate_up [E,2F,H] bf16 ~N(0,1/H) with the
    gate rows first; w_down [E,H,F] bf16 ~N(0,1/F); optional shared expert
    w_gate_up [2Fs,H] ~N(0,1/H), w_down [H,Fs] ~N(0,1/Fs).
    """
    cid: int
    name: str
    T: int
    H: int
    F: int
    E: int
    top_k: int
    padding_m: int
    block_m: int
    rsf: float = 1.0
    zipf_s: Optional[float] = None
    shared_F: int = 0
    scoring: str = "softmax"
    renormalize: bool = True

    @property
    def numel(self) -> int:
        return self.T * self.top_k


@dataclasses.dataclass(frozen=True)
class QuantConfig:
    """Fused SwiGLU + FP8 quantizer workload: x [M, 2F] bf16 ~N(0,1), gate|up halves."""
    cid: int
    name: str
    M: int
    F: int


CONFIGS = {
    "tiny": MoEConfig(0, "tiny", T=64, H=128, F=256, E=8, top_k=2, padding_m=64, block_m=64),
    "qwen3_decode": MoEConfig(1, "qwen3_decode", T=512, H=2048, F=768, E=128, top_k=8,
                              padding_m=128, block_m=128),
    "qwen3_prefill": MoEConfig(2, "qwen3_prefill", T=4096, H=2048, F=768, E=128, top_k=8,
                               padding_m=128, block_m=128),
    "dsv3_prefill": MoEConfig(3, "dsv3_prefill", T=4096, H=7168, F=2048, E=256, top_k=8,
                              padding_m=128, block_m=128, rsf=2.827, zipf_s=1.1, shared_F=2048),
}
# Kimi-K2-scale routed + shared forward (TileOPs #778 "Benchmark": E=384, K=8,
# H=7168, F=2048, F_s=18432, bf16, sigmoid routing) at the token counts of that
# table. One workload id for all of them: the weights are the same tensors and
# each token count's hidden states and logits are the first T rows of the
# T=4096 ones.
KIMI_K2_TOKENS = (1, 32, 512, 2048, 4096)
for _t in KIMI_K2_TOKENS:
    CONFIGS[f"kimi_k2_t{_t}"] = MoEConfig(5, f"kimi_k2_t{_t}", T=_t, H=7168, F=2048, E=384, top_k=8, padding_m=128,
                                          block_m=128, shared_F=18432, scoring="sigmoid")
QUANT_CONFIG = QuantConfig(4, "swiglu_quant_fp8", M=32768, F=2048)
QUANT_EDGE_M = (0, 1, 127, 128, 129)


TAG_GEMM_A, TAG_GEMM_W = 8, 9


@dataclasses.dataclass(frozen=True)
class GemmCase:
    """Aligned grouped GEMM C[e] = A[e] @ B[e]^T over E groups of exactly M rows:
    A [E*M, K] bf16 ~N(0,1) (groups stored one after another), B [E, N, K] bf16
    ~N(0,1/K). The shapes are those of the TileOPs grouped-GEMM baseline table
    (PR #1580, "Benchmark results - grouped-GEMM baselines"), whose cases give the
    rows per expert M and the token count T; E = T / M (rounded down where T is
    not a multiple of M). `page_tflops` is that table's H200 figure for the
    persistent kernel, kept as context."""
    cid: int
    name: str
    M: int
    N: int
    K: int
    E: int
    page_tflops: float


GEMM_CASES = {c.name: c for c in (
    GemmCase(20, "glm5_up_t32768", 1024, 4096, 6144, 32, 599.8),
    GemmCase(21, "glm5_up_t65536", 2048, 4096, 6144, 32, 607.6),
    GemmCase(22, "glm5_up_t131072", 4096, 4096, 6144, 32, 614.8),
    GemmCase(23, "glm5_up_t262144", 8192, 4096, 6144, 32, 612.7),
    GemmCase(24, "glm5_down_t32768", 1024, 6144, 2048, 32, 564.6),
    GemmCase(25, "glm5_down_t65536", 2048, 6144, 2048, 32, 596.3),
    GemmCase(26, "glm5_down_t131072", 4096, 6144, 2048, 32, 603.0),
    GemmCase(27, "glm5_down_t262144", 8192, 6144, 2048, 32, 602.9),
    GemmCase(28, "llama4_128e_up_t131072", 1024, 16384, 5120, 128, 549.9),
    GemmCase(29, "llama4_128e_down_t131072", 1024, 5120, 8192, 128, 604.8),
    GemmCase(30, "qwen3.5_397b_up_t52429", 1024, 2048, 4096, 51, 613.5),
    GemmCase(31, "qwen3.5_397b_down_t52429", 1024, 4096, 1024, 51, 575.8),
)}


def gemm_a(case: GemmCase, device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    """A [E*M, K] (or the given rows of it)."""
    r0, r1 = (0, case.E * case.M) if rows is None else (rows.start, rows.stop)
    return normal_bf16(tensor_key(case.cid, TAG_GEMM_A), (r1 - r0, case.K), 1.0, device, start=r0 * case.K)


def gemm_w(case: GemmCase, device="cpu", experts: Optional[Sequence[int]] = None) -> torch.Tensor:
    """B [E, N, K] (or [len(experts), N, K] for a subset)."""
    per = case.N * case.K
    key = tensor_key(case.cid, TAG_GEMM_W)
    sigma = 1.0 / math.sqrt(case.K)
    if experts is None:
        return normal_bf16(key, (case.E, case.N, case.K), sigma, device)
    return torch.stack([normal_bf16(key, (case.N, case.K), sigma, device, start=e * per) for e in experts])


TAG_GQ_X, TAG_GQ_SIZES = 10, 11


@dataclasses.dataclass(frozen=True)
class GroupedQuantCase:
    """Grouped 1x128-tile FP8 quantizer workload (xtuner #2089, "Single-kernel
    benchmark" and its tests): x [M, K] bf16 ~N(0,1) (gate_up [M, 2K] when
    swiglu), rows in E consecutive expert groups. `sizes` fixes the group
    sizes; otherwise they are a seeded multinomial split of M over E equally
    likely experts (unaligned counts, the pages give no distribution)."""
    cid: int
    name: str
    M: int
    K: int
    E: int
    swiglu: bool = False
    sizes: Optional[tuple] = None


GROUPED_QUANT_CASES = {c.name: c for c in (
    GroupedQuantCase(40, "quant_groups_0_1_127_128_129_k6144", 385, 6144, 5, sizes=(0, 1, 127, 128, 129)),
    GroupedQuantCase(41, "quant_131072x6144_e256", 131072, 6144, 256),
    GroupedQuantCase(42, "swiglu_quant_131072x8192_e256", 131072, 4096, 256, swiglu=True),
)}


def grouped_quant_sizes(case: GroupedQuantCase) -> np.ndarray:
    """int32 [E] group sizes summing to M."""
    if case.sizes is not None:
        return np.asarray(case.sizes, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(tensor_key(case.cid, TAG_GQ_SIZES)))
    return rng.multinomial(case.M, np.full(case.E, 1.0 / case.E)).astype(np.int32)


def grouped_quant_input(case: GroupedQuantCase, device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    """x [M, K] (or [M, 2K] with swiglu), or the given rows of it."""
    w = (2 if case.swiglu else 1) * case.K
    r0, r1 = (0, case.M) if rows is None else (rows.start, rows.stop)
    return normal_bf16(tensor_key(case.cid, TAG_GQ_X), (r1 - r0, w), 1.0, device, start=r0 * w)


def zipf_bias(cfg: MoEConfig) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank), rank a seeded permutation of 1..E (float32)."""
    rng = np.random.Generator(np.random.PCG64(tensor_key(cfg.cid, TAG_BIAS)))
    rank = rng.permutation(cfg.E) + 1
    return (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def hidden(cfg: MoEConfig, device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    r0, r1 = (0, cfg.T) if rows is None else (rows.start, rows.stop)
    return normal_bf16(tensor_key(cfg.cid, TAG_HIDDEN), (r1 - r0, cfg.H), 1.0, device,
                       start=r0 * cfg.H)


def router_logits(cfg: MoEConfig, device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    """Router logits [T, E] float32 from a true N(0, 1) (rows r0..r1-1 of them).

    Unlike the hashed Irwin-Hall stream of the other tensors, the logits keep a
    normal's tails: with a per-expert bias, which experts get any tokens at all
    depends on the rare large logits, and a sum of four uniforms (cut at
    +-3.46 sigma) would starve the experts the bias ranks low. numpy's PCG64
    generator, seeded with SeedSequence([workload id, tensor tag]), draws them
    on the host with `standard_normal(dtype=float32)` (ziggurat), and the bytes
    are uploaded.
    The stream is drawn row-major from its start, so the first T rows are the
    same for every T (a row range is a slice of the rows up to its end).
    """
    r0, r1 = (0, cfg.T) if rows is None else (rows.start, rows.stop)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.cid, TAG_LOGITS])))
    z = rng.standard_normal(r1 * cfg.E, dtype=np.float32).reshape(r1, cfg.E)[r0:r1]
    return torch.from_numpy(np.ascontiguousarray(z)).to(device)


def expert_bias(cfg: MoEConfig, device="cpu") -> Optional[torch.Tensor]:
    """The per-expert Zipf bias [E] float32 of a skewed workload (None without one)."""
    if cfg.zipf_s is None:
        return None
    return torch.from_numpy(zipf_bias(cfg)).to(device)


def w_gate_up(cfg: MoEConfig, device="cpu", experts: Optional[Sequence[int]] = None) -> torch.Tensor:
    """[E,2F,H] (or [len(experts),2F,H] for a subset), gate rows 0..F-1, up rows F..2F-1."""
    per = 2 * cfg.F * cfg.H
    key = tensor_key(cfg.cid, TAG_WGU)
    sigma = 1.0 / math.sqrt(cfg.H)
    if experts is None:
        return normal_bf16(key, (cfg.E, 2 * cfg.F, cfg.H), sigma, device)
    return torch.stack([normal_bf16(key, (2 * cfg.F, cfg.H), sigma, device, start=e * per)
                        for e in experts]) if len(experts) else \
        torch.empty(0, 2 * cfg.F, cfg.H, dtype=torch.bfloat16, device=device)


def w_down(cfg: MoEConfig, device="cpu", experts: Optional[Sequence[int]] = None) -> torch.Tensor:
    """[E,H,F] (or a subset of experts)."""
    per = cfg.H * cfg.F
    key = tensor_key(cfg.cid, TAG_WD)
    sigma = 1.0 / math.sqrt(cfg.F)
    if experts is None:
        return normal_bf16(key, (cfg.E, cfg.H, cfg.F), sigma, device)
    return torch.stack([normal_bf16(key, (cfg.H, cfg.F), sigma, device, start=e * per)
                        for e in experts]) if len(experts) else \
        torch.empty(0, cfg.H, cfg.F, dtype=torch.bfloat16, device=device)


def shared_w_gate_up(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    return normal_bf16(tensor_key(cfg.cid, TAG_SWGU), (2 * cfg.shared_F, cfg.H),
                       1.0 / math.sqrt(cfg.H), device)


def shared_w_down(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    return normal_bf16(tensor_key(cfg.cid, TAG_SWD), (cfg.H, cfg.shared_F),
                       1.0 / math.sqrt(cfg.shared_F), device)


def quant_input(M: int, F: int, device="cpu", rows: Optional[slice] = None,
                cid: int = QUANT_CONFIG.cid) -> torch.Tensor:
    """x [M, 2F] bf16 ~N(0,1): columns 0..F-1 are the gate half, F..2F-1 the up half."""
    r0, r1 = (0, M) if rows is None else (rows.start, rows.stop)
    return normal_bf16(tensor_key(cid, TAG_QUANT, M), (r1 - r0, 2 * F), 1.0, device,
                       start=r0 * 2 * F)
