"""Oracle: a plain, slow host implementation of the routed-expert MoE forward
and the fused SwiGLU + FP8 quantizer, used to check the HIP path.

THIS IS TEST INFRASTRUCTURE. Only the tests, the smoke check of the build
entry point and the benchmark's CPU-baseline leg may import it; the product
library never does, and it shares no code with the HIP kernels.

Every function follows a step as the pages state it (see each docstring for
the page and section); where the pages leave a step open, the docstring says
which reading is taken. Its correctness is pinned independently of itself by
the CPU tests: the tutorial's worked dispatch example, brute-force checks on
tiny inputs, closed forms and library codecs.
"""
from .numerics import (bf16_to_f32, bf16_to_f64, e4m3_decode, e4m3_encode, exp32,
                       round_bf16, silu32, to_bf16)
from .moe import (block_decode, dispatch_tables, forward, grouped_gemm, num_blocks,
                  permute, route, shared_expert, swiglu, unpermute)
from .quant import (block_quant_fp8, expand_128x_starts, grouped_gemm_fp8, quant_fp8, quant_fp8_grouped,
                    swiglu_quant_fp8)

__all__ = [
    "bf16_to_f32", "bf16_to_f64", "e4m3_decode", "e4m3_encode", "exp32", "round_bf16",
    "silu32", "to_bf16", "block_decode", "dispatch_tables", "forward", "grouped_gemm",
    "num_blocks", "permute", "route", "shared_expert", "swiglu", "unpermute", "quant_fp8",
    "swiglu_quant_fp8", "quant_fp8_grouped", "expand_128x_starts", "block_quant_fp8", "grouped_gemm_fp8",
]
