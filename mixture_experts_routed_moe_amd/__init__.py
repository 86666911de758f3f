"""MI355X-native routed-expert MoE forward and fused SwiGLU + FP8 quantizer.

The compute lives in libmoe_mi355x.so (hand-written HIP kernels for gfx950,
C ABI declared in include/moe_mi355x.h); this package is its Python binding.
"""
from ._lib import (EXPORTS, LIB_PATH, MoeError, align_workspace_bytes, alloc_tables, grouped_gemm_down,
                   grouped_gemm_gate_up, grouped_gemm_gate_up_gather, lib, moe_align, moe_align_noalloc, moe_align_noalloc_max_scratch_bytes, moe_permute, moe_topk_softmax, moe_unpermute,
                   num_blocks, swiglu, swiglu_quant_fp8, tile_quant_fp8, tile_quant_fp8_m_pad_bound,
                   fp8_block_quant_weights, grouped_gemm_fp8, grouped_gemm_gate_up_fp8)
from .forward import MoEBuffers, MoEForwardGraph, MoEShape, intermediates, routed_moe_forward

__all__ = [
    "EXPORTS", "LIB_PATH", "MoeError", "align_workspace_bytes", "alloc_tables", "grouped_gemm_down",
    "grouped_gemm_gate_up", "grouped_gemm_gate_up_gather", "lib", "moe_align", "moe_align_noalloc", "moe_align_noalloc_max_scratch_bytes", "moe_permute", "moe_topk_softmax", "moe_unpermute",
    "num_blocks", "swiglu", "swiglu_quant_fp8", "tile_quant_fp8", "tile_quant_fp8_m_pad_bound",
    "fp8_block_quant_weights", "grouped_gemm_fp8", "grouped_gemm_gate_up_fp8", "MoEBuffers", "MoEForwardGraph", "MoEShape", "intermediates",
    "routed_moe_forward",
]
