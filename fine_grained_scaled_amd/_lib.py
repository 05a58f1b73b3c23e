"""ctypes declarations of libfgs's C ABI (include/fgs.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfgs.so")

FGS_OK, FGS_ERR_INVALID_ARG, FGS_ERR_UNSUPPORTED, FGS_ERR_HIP = 0, -1, -2, -3
ELEM_E4M3, ELEM_E2M1, ELEM_E5M2 = 0, 1, 2
SCALE_TENSOR, SCALE_TILE_1x128, SCALE_BLOCK_128x128, SCALE_MX32_E8M0, SCALE_NV16_E4M3 = 0, 1, 2, 3, 4
ROUND_RNE, ROUND_STOCHASTIC = 0, 1
OUT_FP32, OUT_BF16 = 0, 1
TILE_AUTO, TILE_NARROW, TILE_WIDE = 0, 1, 2

EXPORTS = (
    "fgs_quantize_blockwise",
    "fgs_quantize_blockwise_noalloc",
    "fgs_quantize_delayed",
    "fgs_quantize_mx",
    "fgs_quantize_nvfp4",
    "fgs_gemm_block_scaled",
    "fgs_gemm_block_scaled_ex",
    "fgs_gemm_kernel_name",
    "fgs_gemm_block_scaled_fp8mma",
    "fgs_grouped_gemm_block_scaled",
    "fgs_grouped_gemm_block_scaled_fp8mma",
    "fgs_grouped_wgrad_block_scaled_fp8mma",
    "fgs_gemm_block_scaled_fp8out",
    "fgs_grouped_gemm_block_scaled_fp8out",
    "fgs_quantize_grouped_colwise",
    "fgs_grouped_colwise_blocks",
    "fgs_swiglu_quantize_grouped",
    "fgs_grouped_wgrad_block_scaled",
    "fgs_workspace_bytes",
    "fgs_gemm_workspace_bytes",
    "fgs_last_error",
    "fgs_version",
)


class FgsOperand(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("elem", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32),
        ("scales", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_void_p),
    ]


class FgsGemmOptions(ctypes.Structure):
    _fields_ = [
        ("tile", ctypes.c_int32),
        ("fp8_mma", ctypes.c_int32),
        ("q_out", ctypes.c_void_p),
        ("scales_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class FgsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fgs error {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libfgs.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with fine_grained_scaled_amd._build.build() "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t
    lib.fgs_quantize_blockwise.argtypes = [P, I64, I64, I64, I32, P, P, P, P, P, SZ, P]
    lib.fgs_quantize_blockwise_noalloc.argtypes = [P, I64, I64, I64, I32, P, P, P, P, P]
    lib.fgs_quantize_delayed.argtypes = [P, I64, I64, I64, I32, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
    lib.fgs_quantize_mx.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    lib.fgs_quantize_nvfp4.argtypes = [P, I64, I64, I64, I32, U64, I32, U64, P, P, P, P, P, P, SZ, P]
    OP = ctypes.POINTER(FgsOperand)
    lib.fgs_gemm_block_scaled.argtypes = [OP, OP, I64, I64, I64, P, I64, I32, P]
    lib.fgs_gemm_block_scaled_fp8mma.argtypes = [OP, OP, I64, I64, I64, P, I64, I32, P]
    lib.fgs_gemm_block_scaled_ex.argtypes = [OP, OP, I64, I64, I64, P, I64, I32, ctypes.POINTER(FgsGemmOptions), P]
    lib.fgs_gemm_kernel_name.argtypes = [OP, OP, I64, I64, I64, I32, ctypes.POINTER(FgsGemmOptions), ctypes.c_char_p,
                                         SZ]
    lib.fgs_grouped_gemm_block_scaled.argtypes = [OP, OP, P, ctypes.c_int32, I64, I64, I64, P, I64, I32, P]
    lib.fgs_grouped_gemm_block_scaled_fp8mma.argtypes = [OP, OP, P, ctypes.c_int32, I64, I64, I64, P, I64, I32, P]
    lib.fgs_gemm_block_scaled_fp8out.argtypes = [OP, OP, I64, I64, I64, P, I64, P, P, P]
    lib.fgs_grouped_gemm_block_scaled_fp8out.argtypes = [OP, OP, P, ctypes.c_int32, I64, I64, I64, P, I64, P, P, P]
    lib.fgs_quantize_grouped_colwise.argtypes = [P, I64, I64, I64, P, I64, P, ctypes.c_int32, P, P, P, I64, P, P]
    lib.fgs_grouped_colwise_blocks.argtypes = [I64, ctypes.c_int32]
    lib.fgs_swiglu_quantize_grouped.argtypes = [P, I64, I64, I64, P, ctypes.c_int32, P, P, P, P, I64, P, P]
    lib.fgs_grouped_colwise_blocks.restype = I64
    lib.fgs_grouped_wgrad_block_scaled.argtypes = [OP, OP, P, ctypes.c_int32, I64, I64, I64, P, I64, I32, P]
    lib.fgs_grouped_wgrad_block_scaled_fp8mma.argtypes = [OP, OP, P, ctypes.c_int32, I64, I64, I64, P, I64, I32, P]
    lib.fgs_workspace_bytes.argtypes = [I64, I64]
    lib.fgs_workspace_bytes.restype = SZ
    lib.fgs_gemm_workspace_bytes.argtypes = [I32, I64, I64]
    lib.fgs_gemm_workspace_bytes.restype = SZ
    lib.fgs_last_error.restype = ctypes.c_char_p
    lib.fgs_version.restype = ctypes.c_char_p
    for name in ("fgs_quantize_blockwise", "fgs_quantize_blockwise_noalloc", "fgs_quantize_delayed", "fgs_quantize_mx", "fgs_quantize_nvfp4",
                 "fgs_gemm_block_scaled", "fgs_gemm_block_scaled_ex", "fgs_gemm_kernel_name",
                 "fgs_gemm_block_scaled_fp8mma",
                 "fgs_grouped_gemm_block_scaled",
                 "fgs_grouped_gemm_block_scaled_fp8mma", "fgs_grouped_wgrad_block_scaled_fp8mma",
                 "fgs_quantize_grouped_colwise", "fgs_grouped_wgrad_block_scaled",
                 "fgs_swiglu_quantize_grouped", "fgs_gemm_block_scaled_fp8out",
                 "fgs_grouped_gemm_block_scaled_fp8out"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FGS_OK:
        raise FgsError(status, load().fgs_last_error().decode())
