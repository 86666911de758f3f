"""The C-ABI library loads and exports every symbol include/*.h declares.

CPU only: nothing here launches a kernel. The size helpers are host
functions, and the argument checks below all fail before any HIP call.
"""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mixture_experts_routed_moe_amd", "libmoe_mi355x.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mixture_experts_routed_moe_amd import build
        build.build()
    lib = ctypes.CDLL(LIB)
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_num_blocks.restype = ctypes.c_int64
    lib.moe_num_blocks.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.moe_align_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_align_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int]
    return lib


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_align", "moe_permute", "grouped_gemm_gate_up", "swiglu", "grouped_gemm_down",
                     "moe_unpermute", "swiglu_quant_fp8", "moe_topk_softmax"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_python_binding_names_match_header():
    import mixture_experts_routed_moe_amd as m
    assert set(m.EXPORTS) == set(declared_functions())


def test_num_blocks_matches_worked_example(lib):
    # tutorial Example 07: 18 pairs, 4 experts, block = padding = 128 -> 5 blocks
    assert lib.moe_num_blocks(18, 4, 128, 128) == 5
    assert lib.moe_num_blocks(4096 * 8, 256, 128, 128) == 512
    assert lib.moe_num_blocks(100, 3, 64, 128) == 2 + 6
    assert lib.moe_num_blocks(10, 3, 64, 96) == -1
    assert lib.moe_num_blocks(0, 8, 64, 64) == 8
    assert lib.moe_abi_version() == 8


def test_workspace_size(lib):
    assert lib.moe_align_workspace_bytes(32768, 256) == 32 * 256 * 4
    assert lib.moe_align_workspace_bytes(0, 8) == 8 * 4
    assert lib.moe_align_workspace_bytes(1025, 3) == 2 * 3 * 4


def test_argument_errors_return_before_launch(lib):
    c = ctypes
    P = c.c_void_p
    # moe_align: padding not a multiple of block
    lib.moe_align.argtypes = [P, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int] + [P] * 7 + [c.c_size_t, P]
    rc = lib.moe_align(None, 4, 2, 8, 96, 64, *([None] * 7), 0, None)
    assert rc == -1 and b"multiple" in lib.moe_last_error()
    # moe_permute: H not a multiple of 8; T = 0 is a no-op
    lib.moe_permute.argtypes = [P, P, P, c.c_int64, c.c_int, c.c_int, P, P]
    assert lib.moe_permute(None, None, None, 4, 2, 12, None, None) == -1
    assert lib.moe_permute(None, None, None, 0, 2, 16, None, None) == 0
    assert lib.moe_permute(None, None, None, 4, 2, 16, None, None) == -1   # neither permutation table
    # grouped GEMM: unsupported block_m, mixed NULL tables
    lib.grouped_gemm_gate_up.argtypes = [P] * 6 + [c.c_int64] + [c.c_int] * 6 + [P, P]
    assert lib.grouped_gemm_gate_up(None, None, None, None, None, None, 8, 1, 128, 128, 128, 96, 1, None, None) == -2
    assert lib.grouped_gemm_gate_up(None, None, 1, None, None, None, 8, 1, 128, 128, 128, 128, 1, None, None) == -1
    # the gathering gate_up: tables required, numel must be T * top_k; T = 0 is a no-op
    lib.grouped_gemm_gate_up_gather.argtypes = ([P, c.c_int64, P, c.c_int] + [P] * 5 + [c.c_int64] +
                                                [c.c_int] * 6 + [P, P])
    assert lib.grouped_gemm_gate_up_gather(None, 4, None, 2, None, None, None, None, None, 8, 1, 128, 128, 128, 128, 1,
                                           None, None) == -1                        # dense (NULL tables)
    assert b"tables" in lib.moe_last_error()
    assert lib.grouped_gemm_gate_up_gather(None, 4, None, 2, None, 1, 1, 1, 1, 0, 8, 128, 128, 128, 128, 1,
                                           None, None) == -1                        # numel != T * top_k
    assert lib.grouped_gemm_gate_up_gather(None, 0, None, 2, None, 1, 1, 1, 1, 0, 8, 128, 128, 128, 128, 1,
                                           None, None) == 0                         # nothing to do
    # quantizer: F not a multiple of 128; M = 0 is a no-op
    lib.swiglu_quant_fp8.argtypes = [P, c.c_int64, c.c_int] + [P] * 5
    assert lib.swiglu_quant_fp8(None, 4, 100, None, None, None, None, None) == -1
    assert lib.swiglu_quant_fp8(None, 0, 256, None, None, None, None, None) == 0
    # the grouped tile quantizer: sizes, flags and widths are checked before any launch
    lib.tile_quant_fp8.argtypes = [P, c.c_int64, c.c_int, c.c_int, P, c.c_int, c.c_int, c.c_int64] + [P] * 5
    lib.tile_quant_fp8_m_pad_bound.restype = c.c_int64
    lib.tile_quant_fp8_m_pad_bound.argtypes = [c.c_int64, c.c_int]
    assert lib.tile_quant_fp8_m_pad_bound(385, 5) == 128 * (4 + 5)
    assert lib.tile_quant_fp8_m_pad_bound(-1, 5) == -1
    # (16, 32: stand-in q_t / s_t addresses, never dereferenced: every call below fails its checks first)
    assert lib.tile_quant_fp8(None, 4, 100, 0, None, 0, 0, 128, None, None, 16, 32, None) == -1   # K % 128
    assert lib.tile_quant_fp8(None, 4, 128, 0, None, 0, 0, 100, None, None, 16, 32, None) == -1   # m_pad % 128
    assert lib.tile_quant_fp8(None, 300, 128, 0, None, 0, 0, 256, None, None, 16, 32, None) == -1  # m_pad < 384
    assert lib.tile_quant_fp8(None, 4, 128, 2, None, 0, 0, 128, None, None, 16, 32, None) == -1   # swiglu flag
    assert lib.tile_quant_fp8(None, 4, 128, 0, None, 0, 3, 128, None, None, 16, 32, None) == -1   # per_tile flag
    assert lib.tile_quant_fp8(None, 4, 128, 0, 1, 0, 0, 128, None, None, 16, 32, None) == -1      # E < 1 with groups
    assert lib.tile_quant_fp8(None, 4, 128, 0, None, 0, 0, 128, None, None, 16, 32, None) == -1   # null x / q_row
    assert lib.tile_quant_fp8(None, 4, 128, 0, None, 0, 0, 128, None, None, 16, None, None) == -1  # q_t without s_t
    assert b"both" in lib.moe_last_error()
    # row layout only (q_t = s_t = NULL): m_pad and the groups play no part
    assert lib.tile_quant_fp8(None, 4, 128, 0, None, 0, 0, 0, None, None, None, None, None) == -1    # null x / q_row
    assert lib.tile_quant_fp8(None, 0, 128, 0, None, 0, 0, 100, None, None, None, None, None) == 0   # nothing to do
    assert lib.tile_quant_fp8(None, 0, 128, 0, None, 0, 0, 0, None, None, 16, 32, None) == 0         # nothing to do
    # FP8 weight preparation and the block-scaled FP8 grouped GEMM
    lib.fp8_block_quant_weights.argtypes = [P, c.c_int64, c.c_int, P, P, P]
    assert lib.fp8_block_quant_weights(None, 100, 128, None, None, None) == -1     # rows % 128
    assert lib.fp8_block_quant_weights(None, 128, 64, None, None, None) == -1      # K % 128
    assert lib.fp8_block_quant_weights(None, 0, 128, None, None, None) == 0
    lib.grouped_gemm_fp8.argtypes = [P] * 8 + [c.c_int64] + [c.c_int] * 5 + [P, P]
    assert lib.grouped_gemm_fp8(*[None] * 8, 64, 1, 200, 128, 128, 128, None, None) == -1   # N % 128
    assert lib.grouped_gemm_fp8(*[None] * 8, 64, 1, 256, 128, 128, 64, None, None) == -2    # block_m != 128
    assert lib.grouped_gemm_fp8(*[None] * 8, 64, 2, 256, 128, 128, 128, None, None) == -1   # dense needs E=1
    assert lib.grouped_gemm_fp8(*[None] * 8, 0, 1, 256, 128, 128, 128, None, None) == 0
    # 32-bit load offsets: A codes or one group's weight codes of 2^32 bytes are refused
    assert lib.grouped_gemm_fp8(*[None] * 8, 1 << 21, 1, 256, 2048, 128, 128, None, None) == -2   # numel * K
    assert lib.grouped_gemm_fp8(*[None] * 8, 64, 1, 1 << 20, 4096, 128, 128, None, None) == -2    # N * K
    # FP8 gate_up: a_rows must be numel (compact) or numel / top_k (gather); block_m 128 only
    lib.grouped_gemm_gate_up_fp8.argtypes = ([P, P, c.c_int64, P, c.c_int, P, P] + [P] * 4 + [c.c_int64] +
                                             [c.c_int] * 6 + [P, P])
    assert lib.grouped_gemm_gate_up_fp8(None, None, 8, None, 1, None, None, 1, 1, 1, 1, 16, 2, 256, 256, 128, 128, 1,
                                        None, None) == -1        # a_rows != numel without sorted_pair
    assert lib.grouped_gemm_gate_up_fp8(None, None, 8, 16, 2, None, None, 1, 1, 1, 1, 16, 2, 256, 256, 128, 64, 1,
                                        None, None) == -2        # block_m 64
    assert lib.grouped_gemm_gate_up_fp8(None, None, 8, 16, 2, None, None, None, None, None, None, 16, 1, 256, 256,
                                        128, 128, 1, None, None) == -1   # gather without tables
    assert lib.grouped_gemm_gate_up_fp8(None, None, 0, 16, 2, None, None, 1, 1, 1, 1, 0, 2, 256, 256, 128, 128, 1,
                                        None, None) == 0         # nothing to do
    assert lib.grouped_gemm_gate_up_fp8(None, None, 1 << 20, None, 1, None, None, None, None, None, None, 1 << 20, 1,
                                        4096, 256, 128, 128, 1, None, None) == -2   # a_rows * H reaches 2^32
    # routing limits
    lib.moe_topk_softmax.argtypes = [P, P, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int, P, P, P]
    assert lib.moe_topk_softmax(None, None, 4, 2048, 8, 0, 1, None, None, None) == -2
    assert lib.moe_topk_softmax(None, None, 4, 8, 9, 0, 1, None, None, None) == -2
    assert lib.moe_topk_softmax(None, None, 4, 8, 2, 2, 1, None, None, None) == -1   # unknown scoring
    assert lib.moe_topk_softmax(None, None, 4, 8, 2, 1, 3, None, None, None) == -1   # renormalize not 0/1
    assert lib.moe_topk_softmax(None, None, 0, 8, 2, 1, 0, None, None, None) == 0    # T = 0: nothing to do
    assert lib.moe_topk_softmax(None, None, 4, 8, 2, 0, 1, None, None, None) == -1   # null pointers
    # unpermute aliasing and null pointers
    lib.moe_unpermute.argtypes = [P, P, P, c.c_int64, c.c_int, c.c_int, c.c_float, P, P, P]
    assert lib.moe_unpermute(None, None, None, 4, 2, 16, 1.0, None, None, None) == -1
