"""fine_grained_scaled_amd: fine-grained scaled FP8/FP4 quantization and
block-scaled GEMM for AMD Instinct MI355X (gfx950), behind a C-ABI library."""
