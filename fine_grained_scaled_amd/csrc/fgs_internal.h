// fgs_internal.h -- launcher interfaces between the C ABI layer and the
// gfx950 kernels of libfgs (validated arguments only reach these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fgs.h"

namespace fgs {

struct QuantE4M3Args {
    const void* x;
    int64_t rows, cols, ldx;
    int mode;
    uint8_t* q;
    float* scales;
    uint8_t* qT;
    float* scalesT;
    void* workspace;   // TENSOR mode: one uint32 amax partial per amax workgroup
    size_t workspace_bytes;
};
hipError_t launch_quant_e4m3(const QuantE4M3Args& a, hipStream_t stream);

// The library's own device scratch for the per-tensor amax partials on the
// current device (a fixed 4 KiB array per device, its address resolved once
// per device): the workspace of fgs_quantize_blockwise_noalloc.
hipError_t quant_scratch(void** ptr, size_t* bytes);

// Per-group column-wise 1x128 quantization (plus the optional row-wise
// output of the grouped rows), TILE mode only.
struct QuantGroupedArgs {
    const void* x;
    int64_t rows, cols, ldx;        // rows: of the (gathered) matrix the groups index
    const int32_t* row_index;       // device int32 [rows] into x, or nullptr (identity)
    int64_t src_rows;               // rows of x when row_index is given
    const int32_t* group_offsets;   // device int32 [G + 1]
    int32_t G;
    uint8_t* q;
    float* scales;
    uint8_t* qT;
    int64_t ldqT;
    float* scalesT;
    int swiglu;                     // x is a gate/up output [rows x 2*cols]; quantize its SwiGLU
    uint16_t* h_out;                // swiglu: optional BF16 activation [rows x cols]
};
hipError_t launch_quant_grouped_colwise(const QuantGroupedArgs& a, hipStream_t stream);

// Per-tensor delayed scaling (E4M3 or E5M2) from an amax history.
struct QuantDelayedArgs {
    const void* x;
    int64_t rows, cols, ldx;
    int elem;                       // FGS_ELEM_E4M3 | FGS_ELEM_E5M2
    float* history;                 // device FP32 [history_len]
    int32_t history_len, slot;
    uint8_t* q;
    uint8_t* qT;
    float* scale;                   // device FP32 [1]
};
hipError_t launch_quant_delayed(const QuantDelayedArgs& a, hipStream_t stream);

struct QuantMXArgs {
    const void* x;
    int64_t rows, cols, ldx;
    uint8_t* q;
    uint8_t* scales;
    uint8_t* qT;
    uint8_t* scalesT;
};
hipError_t launch_quant_mx(const QuantMXArgs& a, hipStream_t stream);

struct QuantNVFP4Args {
    const void* x;
    int64_t rows, cols, ldx;
    int rht_mask;
    uint64_t rht_seed;
    int stochastic;
    uint64_t sr_seed;
    uint8_t* q;
    uint8_t* scales;
    uint8_t* qT;
    uint8_t* scalesT;
    float* tensor_scale;
    void* workspace;   // two uint32 amax partials per amax workgroup
    size_t workspace_bytes;
};
hipError_t launch_quant_nvfp4(const QuantNVFP4Args& a, hipStream_t stream);

struct GemmArgs {
    fgs_operand A, B;
    int64_t M, N, K;
    void* C;
    int64_t ldc;
    int out_bf16;
    // grouped variants
    const int32_t* group_offsets;   // nullptr for the dense GEMM
    int32_t G;
    int group_k;                    // groups split the contraction (MoE wgrad)
    int64_t T;                      // group_k: tokens the offsets index
    uint8_t* q_out;                 // BF16 out: also 1x128 E4M3 codes of the output, or nullptr
    float* s_out;                   //   their scales [N/128][M]
    int fp8_mma;                    // accumulate on the FP8 matrix instructions
    int tile;                       // dense only: FGS_TILE_AUTO | FGS_TILE_NARROW | FGS_TILE_WIDE
    char* name_out;                 // non-null: write the kernel instantiation's name instead of launching
    size_t name_len;
    void* workspace;                // MXFP8 exact path: 2 (M + N) bytes for the rows' references, or nullptr
};
// Compute units of the current device (cached per device; 256 if the
// query fails).
int device_cus();

hipError_t launch_gemm_fp8(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_nvfp4(const GemmArgs& a, hipStream_t stream);

} // namespace fgs
