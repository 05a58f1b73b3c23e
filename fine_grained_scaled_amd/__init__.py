"""fine_grained_scaled_amd: fine-grained scaled FP8/FP4 quantization and
block-scaled GEMM for AMD Instinct MI355X (gfx950), behind the C ABI of
libfgs (include/fgs.h).  The Python layer only marshals arguments."""
from ._lib import (ELEM_E2M1, ELEM_E4M3, ELEM_E5M2, SCALE_BLOCK_128x128, SCALE_MX32_E8M0, SCALE_NV16_E4M3,
                   SCALE_TENSOR, SCALE_TILE_1x128, FgsError)
from .linear import DelayedState, Linear, fp8_linear
from .ops import (Operand, Quantized, gemm_block_scaled, gemm_block_scaled_fp8out, gemm_kernel_name,
                  grouped_colwise_blocks, grouped_gemm_block_scaled, grouped_gemm_block_scaled_fp8out, grouped_wgrad_block_scaled, quantize_blockwise,
                  quantize_delayed, quantize_grouped_colwise, quantize_mx, quantize_nvfp4,
                  swiglu_quantize_grouped)

__all__ = [
    "Linear", "fp8_linear", "DelayedState",
    "gemm_block_scaled_fp8out", "grouped_gemm_block_scaled_fp8out", "gemm_kernel_name",
    "quantize_blockwise", "quantize_delayed", "quantize_mx", "quantize_nvfp4", "gemm_block_scaled",
    "grouped_gemm_block_scaled", "quantize_grouped_colwise", "grouped_colwise_blocks",
    "grouped_wgrad_block_scaled", "swiglu_quantize_grouped", "Operand", "Quantized", "FgsError",
    "ELEM_E4M3", "ELEM_E2M1", "ELEM_E5M2", "SCALE_TENSOR", "SCALE_TILE_1x128", "SCALE_BLOCK_128x128",
    "SCALE_MX32_E8M0", "SCALE_NV16_E4M3",
]
