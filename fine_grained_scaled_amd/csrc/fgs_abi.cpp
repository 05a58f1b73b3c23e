// fgs_abi.cpp -- the extern "C" entry points of libfgs: argument validation
// (before any HIP call), error reporting, and dispatch to the launchers.
// The operations themselves are documented in include/fgs.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "fgs_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok()
{
    g_last_error.clear();
    return FGS_OK;
}

int hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ok();
    return fail(FGS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxRowBlocks = 65535;   // grid.y limit of the 128x128 quant kernels
// the grouped quantizers launch the column blocks along grid.x and the
// token blocks along grid.y
constexpr int64_t kMaxColBlocks = 0x7FFFFFFF;

int check_bf16_source(const void* x, int64_t rows, int64_t cols, int64_t ldx)
{
    if (rows < 0 || cols < 0) return fail(FGS_ERR_INVALID_ARG, "rows (%lld) and cols (%lld) must be >= 0",
                                          (long long)rows, (long long)cols);
    if (rows == 0 || cols == 0) return FGS_OK;
    if (!x) return fail(FGS_ERR_INVALID_ARG, "x is NULL");
    if (ldx < cols) return fail(FGS_ERR_INVALID_ARG, "ldx (%lld) < cols (%lld)", (long long)ldx, (long long)cols);
    if (cols % 8 || ldx % 8) return fail(FGS_ERR_UNSUPPORTED, "cols and ldx must be multiples of 8 (16-byte rows)");
    if (!aligned(x, 16)) return fail(FGS_ERR_UNSUPPORTED, "x must be 16-byte aligned");
    if ((rows + 127) / 128 > kMaxRowBlocks) return fail(FGS_ERR_UNSUPPORTED, "rows too large (%lld)", (long long)rows);
    return FGS_OK;
}

int check_operand(const fgs_operand* op, const char* name, int64_t rows, int64_t K)
{
    if (!op) return fail(FGS_ERR_INVALID_ARG, "%s is NULL", name);
    if (rows == 0) return FGS_OK;
    if (!op->data) return fail(FGS_ERR_INVALID_ARG, "%s.data is NULL", name);
    if (!op->scales) return fail(FGS_ERR_INVALID_ARG, "%s.scales is NULL", name);
    if (op->ld < K) return fail(FGS_ERR_INVALID_ARG, "%s.ld (%lld) < K (%lld)", name, (long long)op->ld, (long long)K);
    const int64_t ld_bytes = op->elem == FGS_ELEM_E2M1 ? op->ld / 2 : op->ld;
    if (op->elem == FGS_ELEM_E2M1 && (op->ld & 1)) return fail(FGS_ERR_UNSUPPORTED, "%s.ld must be even for E2M1", name);
    if (ld_bytes % 16) return fail(FGS_ERR_UNSUPPORTED, "%s row stride must be a multiple of 16 bytes", name);
    // the GEMM addresses a tile's rows by 32-bit offsets from its first row
    if (ld_bytes >= ((int64_t)1 << 24)) return fail(FGS_ERR_UNSUPPORTED, "%s row stride must be below 2^24 bytes", name);
    if (!aligned(op->data, 16)) return fail(FGS_ERR_UNSUPPORTED, "%s.data must be 16-byte aligned", name);
    if (!aligned(op->scales, 4)) return fail(FGS_ERR_UNSUPPORTED, "%s.scales must be 4-byte aligned", name);
    return FGS_OK;
}

} // namespace

namespace fgs {

// A per-thread memo of a device property (no state shared between threads
// or carried from one call's arguments into another's behaviour).
int device_cus()
{
    thread_local int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev];
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return n;
}

} // namespace fgs

extern "C" {

const char* fgs_last_error(void) { return g_last_error.c_str(); }

const char* fgs_version(void) { return "fgs 0.1.0 (gfx950)"; }

// The tensor-amax passes keep one partial per amax workgroup (4 bytes for
// TENSOR mode, 8 for NVFP4's two orientations), up to two workgroups per
// compute unit: 4 KiB covers 256 compute units at full speed.
size_t fgs_gemm_workspace_bytes(int a_scale_mode, int64_t M, int64_t N)
{
    if (a_scale_mode != FGS_SCALE_MX32_E8M0 || M < 0 || N < 0) return 0;
    return (size_t)(2 * (M + N));
}

size_t fgs_workspace_bytes(int64_t rows, int64_t cols)
{
    (void)rows;
    (void)cols;
    return 4096;
}

// Arguments of fgs_quantize_blockwise apart from its workspace.
static int check_blockwise(const void* x, int64_t rows, int64_t cols, int64_t ldx, int mode,
                           uint8_t* q, float* scales, uint8_t* qT, float* scalesT)
{
    if (mode != FGS_SCALE_TENSOR && mode != FGS_SCALE_TILE_1x128 && mode != FGS_SCALE_BLOCK_128x128)
        return fail(FGS_ERR_INVALID_ARG, "mode %d is not TENSOR, TILE_1x128 or BLOCK_128x128", mode);
    int st = check_bf16_source(x, rows, cols, ldx);
    if (st != FGS_OK) return st;
    if (rows == 0 || cols == 0 || (!q && !qT)) return FGS_OK;
    if (q) {
        if (!scales) return fail(FGS_ERR_INVALID_ARG, "scales is NULL while q is given");
        if (cols % 128) return fail(FGS_ERR_UNSUPPORTED, "row-wise output needs cols %% 128 == 0 (cols = %lld)", (long long)cols);
        if (!aligned(q, 16) || !aligned(scales, 4)) return fail(FGS_ERR_UNSUPPORTED, "q must be 16-byte and scales 4-byte aligned");
    }
    if (qT) {
        if (!scalesT && mode != FGS_SCALE_TENSOR) return fail(FGS_ERR_INVALID_ARG, "scalesT is NULL while qT is given");
        if (rows % 128) return fail(FGS_ERR_UNSUPPORTED, "column-wise output needs rows %% 128 == 0 (rows = %lld)", (long long)rows);
        if (!aligned(qT, 16) || (scalesT && !aligned(scalesT, 4))) return fail(FGS_ERR_UNSUPPORTED, "qT must be 16-byte and scalesT 4-byte aligned");
    }
    return FGS_OK;
}

int fgs_quantize_blockwise(const void* x, int64_t rows, int64_t cols, int64_t ldx, int mode,
                           uint8_t* q, float* scales, uint8_t* qT, float* scalesT,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_blockwise(x, rows, cols, ldx, mode, q, scales, qT, scalesT);
    if (st != FGS_OK) return st;
    if (rows == 0 || cols == 0 || (!q && !qT)) return ok();
    if (mode == FGS_SCALE_TENSOR) {
        if (!workspace || workspace_bytes < 4) return fail(FGS_ERR_INVALID_ARG, "TENSOR mode needs a workspace of >= 4 bytes");
        if (!aligned(workspace, 4)) return fail(FGS_ERR_UNSUPPORTED, "workspace must be 4-byte aligned");
    }
    fgs::QuantE4M3Args a{x, rows, cols, ldx, mode, q, scales, qT, scalesT, workspace, workspace_bytes};
    return hip_status(fgs::launch_quant_e4m3(a, static_cast<hipStream_t>(stream)), "quantize_blockwise launch");
}

int fgs_quantize_blockwise_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ldx, int mode,
                                   uint8_t* q, float* scales, uint8_t* qT, float* scalesT, void* stream)
{
    int st = check_blockwise(x, rows, cols, ldx, mode, q, scales, qT, scalesT);
    if (st != FGS_OK) return st;
    if (rows == 0 || cols == 0 || (!q && !qT)) return ok();
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (mode == FGS_SCALE_TENSOR) {
        // the library's own 4 KiB per device: the amax pass runs at most one
        // workgroup per 4-byte slot, so every input size fits it
        hipError_t e = fgs::quant_scratch(&ws, &ws_bytes);
        if (e != hipSuccess) return hip_status(e, "quantize_blockwise_noalloc: scratch address");
        if (ws_bytes < 4) return fail(FGS_ERR_UNSUPPORTED, "scratch of %zu bytes is below one amax slot", ws_bytes);
    }
    fgs::QuantE4M3Args a{x, rows, cols, ldx, mode, q, scales, qT, scalesT, ws, ws_bytes};
    return hip_status(fgs::launch_quant_e4m3(a, static_cast<hipStream_t>(stream)), "quantize_blockwise_noalloc launch");
}

int fgs_quantize_delayed(const void* x, int64_t rows, int64_t cols, int64_t ldx, int elem,
                         float* amax_history, int32_t history_len, int32_t slot,
                         uint8_t* q, uint8_t* qT, float* scale, void* stream)
{
    if (elem != FGS_ELEM_E4M3 && elem != FGS_ELEM_E5M2)
        return fail(FGS_ERR_INVALID_ARG, "elem %d is not E4M3 or E5M2", elem);
    int st = check_bf16_source(x, rows, cols, ldx);
    if (st != FGS_OK) return st;
    if (!amax_history || !aligned(amax_history, 4)) return fail(FGS_ERR_INVALID_ARG, "amax_history must be a 4-byte aligned device pointer");
    if (history_len < 1 || history_len > 65536) return fail(FGS_ERR_INVALID_ARG, "history_len (%d) must be in 1..65536", history_len);
    if (slot < 0 || slot >= history_len) return fail(FGS_ERR_INVALID_ARG, "slot (%d) must be in [0, history_len)", slot);
    if (!scale || !aligned(scale, 4)) return fail(FGS_ERR_INVALID_ARG, "scale must be a 4-byte aligned device pointer");
    if (q && !aligned(q, 16)) return fail(FGS_ERR_UNSUPPORTED, "q must be 16-byte aligned");
    if (qT) {
        if (rows % 128) return fail(FGS_ERR_UNSUPPORTED, "column-wise output needs rows %% 128 == 0 (rows = %lld)", (long long)rows);
        if (!aligned(qT, 16)) return fail(FGS_ERR_UNSUPPORTED, "qT must be 16-byte aligned");
    }
    fgs::QuantDelayedArgs a{x, rows, cols, ldx, elem, amax_history, history_len, slot, q, qT, scale};
    return hip_status(fgs::launch_quant_delayed(a, static_cast<hipStream_t>(stream)), "quantize_delayed launch");
}

int fgs_quantize_mx(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                    uint8_t* q, uint8_t* scales, uint8_t* qT, uint8_t* scalesT, void* stream)
{
    int st = check_bf16_source(x, rows, cols, ldx);
    if (st != FGS_OK) return st;
    if (rows == 0 || cols == 0 || (!q && !qT)) return ok();
    if (q) {
        if (!scales) return fail(FGS_ERR_INVALID_ARG, "scales is NULL while q is given");
        if (cols % 32) return fail(FGS_ERR_UNSUPPORTED, "row-wise output needs cols %% 32 == 0");
        if (!aligned(q, 16)) return fail(FGS_ERR_UNSUPPORTED, "q must be 16-byte aligned");
    }
    if (qT) {
        if (!scalesT) return fail(FGS_ERR_INVALID_ARG, "scalesT is NULL while qT is given");
        if (rows % 128) return fail(FGS_ERR_UNSUPPORTED, "column-wise output needs rows %% 128 == 0");
        if (!aligned(qT, 16)) return fail(FGS_ERR_UNSUPPORTED, "qT must be 16-byte aligned");
    }
    fgs::QuantMXArgs a{x, rows, cols, ldx, q, scales, qT, scalesT};
    return hip_status(fgs::launch_quant_mx(a, static_cast<hipStream_t>(stream)), "quantize_mx launch");
}

int fgs_quantize_nvfp4(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                       int rht_mask, uint64_t rht_seed, int round, uint64_t sr_seed,
                       uint8_t* q, uint8_t* scales, uint8_t* qT, uint8_t* scalesT,
                       float* tensor_scale, void* workspace, size_t workspace_bytes, void* stream)
{
    if (rht_mask < 0 || rht_mask > 3) return fail(FGS_ERR_INVALID_ARG, "rht_mask must be in 0..3");
    if (round != FGS_ROUND_RNE && round != FGS_ROUND_STOCHASTIC) return fail(FGS_ERR_INVALID_ARG, "round must be RNE or STOCHASTIC");
    int st = check_bf16_source(x, rows, cols, ldx);
    if (st != FGS_OK) return st;
    if (rows == 0 || cols == 0 || (!q && !qT)) return ok();
    if (!tensor_scale || !aligned(tensor_scale, 4)) return fail(FGS_ERR_INVALID_ARG, "tensor_scale must be a 4-byte aligned device pointer");
    if (!workspace || workspace_bytes < 8 || !aligned(workspace, 4)) return fail(FGS_ERR_INVALID_ARG, "NVFP4 needs a workspace of >= 8 bytes");
    if (q) {
        if (!scales) return fail(FGS_ERR_INVALID_ARG, "scales is NULL while q is given");
        if (cols % 16) return fail(FGS_ERR_UNSUPPORTED, "row-wise output needs cols %% 16 == 0");
        if (!aligned(q, 16)) return fail(FGS_ERR_UNSUPPORTED, "q must be 16-byte aligned");
    }
    if (qT) {
        if (!scalesT) return fail(FGS_ERR_INVALID_ARG, "scalesT is NULL while qT is given");
        if (rows % 128) return fail(FGS_ERR_UNSUPPORTED, "column-wise output needs rows %% 128 == 0");
        if (!aligned(qT, 16)) return fail(FGS_ERR_UNSUPPORTED, "qT must be 16-byte aligned");
    }
    fgs::QuantNVFP4Args a{x, rows, cols, ldx, rht_mask, rht_seed, round == FGS_ROUND_STOCHASTIC, sr_seed,
                          q, scales, qT, scalesT, tensor_scale, workspace, workspace_bytes};
    return hip_status(fgs::launch_quant_nvfp4(a, static_cast<hipStream_t>(stream)), "quantize_nvfp4 launch");
}

static int check_gemm_common(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                             void* C, int64_t ldc, int out_dtype)
{
    if (M < 0 || N < 0 || K < 0) return fail(FGS_ERR_INVALID_ARG, "M, N, K must be >= 0");
    if (out_dtype != FGS_OUT_FP32 && out_dtype != FGS_OUT_BF16) return fail(FGS_ERR_INVALID_ARG, "out_dtype %d invalid", out_dtype);
    if (!A || !B) return fail(FGS_ERR_INVALID_ARG, "A and B must not be NULL");
    if (M == 0 || N == 0) return FGS_OK;
    if (K == 0 || K % 128) return fail(FGS_ERR_UNSUPPORTED, "K must be a positive multiple of 128 (K = %lld)", (long long)K);
    if (!C) return fail(FGS_ERR_INVALID_ARG, "C is NULL");
    if (ldc < N) return fail(FGS_ERR_INVALID_ARG, "ldc (%lld) < N (%lld)", (long long)ldc, (long long)N);
    if (!aligned(C, out_dtype == FGS_OUT_FP32 ? 4 : 2)) return fail(FGS_ERR_UNSUPPORTED, "C misaligned");
    for (const fgs_operand* op : {A, B})
        if (op->elem != FGS_ELEM_E4M3 && op->elem != FGS_ELEM_E2M1 && op->elem != FGS_ELEM_E5M2)
            return fail(FGS_ERR_INVALID_ARG, "unknown element format %d", op->elem);
    const bool fp8 = [](int e) { return e == FGS_ELEM_E4M3 || e == FGS_ELEM_E5M2; }(A->elem) &&
                     (B->elem == FGS_ELEM_E4M3 || B->elem == FGS_ELEM_E5M2);
    if (A->elem != B->elem && !fp8) return fail(FGS_ERR_UNSUPPORTED, "A and B element formats differ");
    if ((A->elem == FGS_ELEM_E5M2 || B->elem == FGS_ELEM_E5M2) &&
        (A->scale_mode != FGS_SCALE_TENSOR || B->scale_mode != FGS_SCALE_TENSOR))
        return fail(FGS_ERR_UNSUPPORTED, "E5M2 operands take per-tensor (TENSOR) scales on both sides");
    int st = check_operand(A, "A", M, K);
    if (st != FGS_OK) return st;
    return check_operand(B, "B", N, K);
}

static bool is_fp32_mode(int m)
{
    return m == FGS_SCALE_TENSOR || m == FGS_SCALE_TILE_1x128 || m == FGS_SCALE_BLOCK_128x128;
}

static int gemm_impl(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                     void* C, int64_t ldc, int out_dtype, const fgs_gemm_options& o, void* stream,
                     char* name = nullptr, size_t name_len = 0)
{
    if (o.tile != FGS_TILE_AUTO && o.tile != FGS_TILE_NARROW && o.tile != FGS_TILE_WIDE)
        return fail(FGS_ERR_INVALID_ARG, "tile %d is not FGS_TILE_AUTO, FGS_TILE_NARROW or FGS_TILE_WIDE", o.tile);
    if (o.fp8_mma != 0 && o.fp8_mma != 1) return fail(FGS_ERR_INVALID_ARG, "fp8_mma must be 0 or 1 (got %d)", o.fp8_mma);
    uint8_t* q_out = o.q_out;
    float* s_out = o.scales_out;
    if (q_out || s_out) {
        // the E4M3-output epilogue: BF16 accumulation output, C optional,
        // codes and scales need N % 128 == 0
        if (!q_out || !s_out) return fail(FGS_ERR_INVALID_ARG, "q_out and scales_out are required together");
        if (out_dtype != FGS_OUT_BF16) return fail(FGS_ERR_INVALID_ARG, "the E4M3 output needs out_dtype FGS_OUT_BF16");
        if (o.fp8_mma) return fail(FGS_ERR_UNSUPPORTED, "the E4M3 output is not available on the FP8 matrix instructions");
        if (N % 128) return fail(FGS_ERR_UNSUPPORTED, "the E4M3 output needs N %% 128 == 0 (N = %lld)", (long long)N);
        if (!aligned(q_out, 4) || !aligned(s_out, 4)) return fail(FGS_ERR_UNSUPPORTED, "q_out and scales_out must be 4-byte aligned");
        if (!C) ldc = N;      // no BF16 output: the common checks see a valid stride
    }
    int st = check_gemm_common(A, B, M, N, K, C ? C : static_cast<void*>(q_out), ldc, out_dtype);
    if (st != FGS_OK) return st;
    if (M == 0 || N == 0) {
        if (name) name[0] = '\0';      // nothing would be launched
        return ok();
    }
    if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30) return fail(FGS_ERR_UNSUPPORTED, "M or N too large");
    // the launch numbers its workgroup tiles (256 x 128 at the finest) in 32 bits
    if (((M + 255) / 256) * ((N + 127) / 128) > 0x7FFFFFFF) return fail(FGS_ERR_UNSUPPORTED, "too many tiles");
    void* ws = nullptr;
    if (o.workspace || o.workspace_bytes) {
        const size_t need = fgs_gemm_workspace_bytes(A->scale_mode, M, N);
        if (!o.workspace || o.workspace_bytes < need)
            return fail(FGS_ERR_INVALID_ARG, "workspace_bytes (%zu) < fgs_gemm_workspace_bytes (%zu), or workspace is NULL",
                        o.workspace_bytes, need);
        if (!aligned(o.workspace, 16)) return fail(FGS_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        if (need > 0) ws = o.workspace;
    }
    fgs::GemmArgs a{*A, *B, M, N, K, C, ldc, out_dtype == FGS_OUT_BF16, nullptr, 0, 0, 0, q_out, s_out, o.fp8_mma,
                    o.tile, name, name_len, ws};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (o.fp8_mma && (A->elem == FGS_ELEM_E2M1 || B->elem == FGS_ELEM_E2M1))
        return fail(FGS_ERR_UNSUPPORTED, "the FP8 matrix-instruction GEMM takes E4M3 / E5M2 operands only");
    if (A->elem != FGS_ELEM_E2M1 && is_fp32_mode(A->scale_mode) && is_fp32_mode(B->scale_mode)) {
        if (A->scale_mode == FGS_SCALE_BLOCK_128x128)
            return fail(FGS_ERR_UNSUPPORTED, "A with 128x128 block scales is not supported (use TILE_1x128 or TENSOR)");
        return hip_status(fgs::launch_gemm_fp8(a, s), "gemm_block_scaled launch");
    }
    if (A->elem == FGS_ELEM_E4M3 && A->scale_mode == FGS_SCALE_MX32_E8M0 && B->scale_mode == FGS_SCALE_MX32_E8M0)
        return hip_status(fgs::launch_gemm_mx(a, s), "gemm_block_scaled (MX) launch");
    if (A->elem == FGS_ELEM_E2M1 && A->scale_mode == FGS_SCALE_NV16_E4M3 && B->scale_mode == FGS_SCALE_NV16_E4M3) {
        if (!A->tensor_scale || !B->tensor_scale) return fail(FGS_ERR_INVALID_ARG, "NVFP4 operands need tensor_scale");
        return hip_status(fgs::launch_gemm_nvfp4(a, s), "gemm_block_scaled (NVFP4) launch");
    }
    return fail(FGS_ERR_UNSUPPORTED, "unsupported operand combination (elem %d, A scale %d, B scale %d)",
                A->elem, A->scale_mode, B->scale_mode);
}

int fgs_gemm_block_scaled_ex(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                             void* C, int64_t ldc, int out_dtype, const fgs_gemm_options* opts, void* stream)
{
    const fgs_gemm_options o = opts ? *opts : fgs_gemm_options{};
    return gemm_impl(A, B, M, N, K, C, ldc, out_dtype, o, stream);
}

int fgs_gemm_kernel_name(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                         int out_dtype, const fgs_gemm_options* opts, char* name, size_t len)
{
    if (!name || len < 2) return fail(FGS_ERR_INVALID_ARG, "name must hold at least 2 bytes");
    const fgs_gemm_options o = opts ? *opts : fgs_gemm_options{};
    // validated as the launch would be, with a stand-in output address that
    // is never written (nothing is launched)
    void* c_stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
    const int st = gemm_impl(A, B, M, N, K, o.q_out ? nullptr : c_stand_in, N, out_dtype, o, nullptr, name, len);
    if (st != FGS_OK) name[0] = '\0';
    return st;
}

int fgs_gemm_block_scaled(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                          void* C, int64_t ldc, int out_dtype, void* stream)
{
    return gemm_impl(A, B, M, N, K, C, ldc, out_dtype, fgs_gemm_options{}, stream);
}

int fgs_gemm_block_scaled_fp8mma(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                                 void* C, int64_t ldc, int out_dtype, void* stream)
{
    fgs_gemm_options o{};
    o.fp8_mma = 1;
    return gemm_impl(A, B, M, N, K, C, ldc, out_dtype, o, stream);
}

// E4M3-output launches: validated like the BF16-out GEMM (C may be NULL);
// the codes and scales need N % 128 == 0.
static int check_fp8_out(int64_t N, void*& C, int64_t& ldc, uint8_t* q_out, float* s_out)
{
    if (!q_out || !s_out) return fail(FGS_ERR_INVALID_ARG, "q_out and scales_out are required");
    if (N % 128) return fail(FGS_ERR_UNSUPPORTED, "the E4M3 output needs N %% 128 == 0 (N = %lld)", (long long)N);
    if (!aligned(q_out, 4) || !aligned(s_out, 4)) return fail(FGS_ERR_UNSUPPORTED, "q_out and scales_out must be 4-byte aligned");
    if (!C) ldc = N;      // no BF16 output: the common checks see a valid stride
    return FGS_OK;
}

int fgs_gemm_block_scaled_fp8out(const fgs_operand* A, const fgs_operand* B, int64_t M, int64_t N, int64_t K,
                                 void* C, int64_t ldc, uint8_t* q_out, float* scales_out, void* stream)
{
    if (!q_out || !scales_out) return fail(FGS_ERR_INVALID_ARG, "q_out and scales_out are required");
    fgs_gemm_options o{};
    o.q_out = q_out;
    o.scales_out = scales_out;
    return gemm_impl(A, B, M, N, K, C, ldc, FGS_OUT_BF16, o, stream);
}

static int grouped_impl(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets, int32_t G,
                        int64_t total_M, int64_t N, int64_t K, void* C, int64_t ldc, int out_dtype,
                        uint8_t* q_out, float* s_out, void* stream, bool fp8_mma = false)
{
    if (G < 0) return fail(FGS_ERR_INVALID_ARG, "G must be >= 0");
    int st = check_gemm_common(A, B, total_M, N, K, C ? C : static_cast<void*>(q_out), ldc, out_dtype);
    if (st != FGS_OK) return st;
    if (total_M == 0 || N == 0 || G == 0) return ok();
    if (!group_offsets) return fail(FGS_ERR_INVALID_ARG, "group_offsets is NULL");
    if (A->elem != FGS_ELEM_E4M3 || A->scale_mode != FGS_SCALE_TILE_1x128 || B->scale_mode != FGS_SCALE_BLOCK_128x128)
        return fail(FGS_ERR_UNSUPPORTED, "grouped GEMM supports E4M3 A TILE_1x128 x B BLOCK_128x128");
    if (total_M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30)) return fail(FGS_ERR_UNSUPPORTED, "sizes too large");
    const int64_t tiles = ((total_M + 127) / 128 + G) * ((N + 127) / 128);
    if (tiles > 0x7FFFFFFF) return fail(FGS_ERR_UNSUPPORTED, "too many tiles");
    fgs::GemmArgs a{*A, *B, total_M, N, K, C, ldc, out_dtype == FGS_OUT_BF16, group_offsets, G, 0, 0, q_out, s_out,
                    fp8_mma ? 1 : 0, FGS_TILE_AUTO};
    return hip_status(fgs::launch_gemm_fp8(a, static_cast<hipStream_t>(stream)), "grouped_gemm_block_scaled launch");
}

int fgs_grouped_gemm_block_scaled(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets,
                                  int32_t G, int64_t total_M, int64_t N, int64_t K,
                                  void* C, int64_t ldc, int out_dtype, void* stream)
{
    return grouped_impl(A, B, group_offsets, G, total_M, N, K, C, ldc, out_dtype, nullptr, nullptr, stream);
}

int fgs_grouped_gemm_block_scaled_fp8mma(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets,
                                         int32_t G, int64_t total_M, int64_t N, int64_t K,
                                         void* C, int64_t ldc, int out_dtype, void* stream)
{
    return grouped_impl(A, B, group_offsets, G, total_M, N, K, C, ldc, out_dtype, nullptr, nullptr, stream, true);
}

int fgs_grouped_gemm_block_scaled_fp8out(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets,
                                         int32_t G, int64_t total_M, int64_t N, int64_t K, void* C, int64_t ldc,
                                         uint8_t* q_out, float* scales_out, void* stream)
{
    int st = check_fp8_out(N, C, ldc, q_out, scales_out);
    if (st != FGS_OK) return st;
    return grouped_impl(A, B, group_offsets, G, total_M, N, K, C, ldc, FGS_OUT_BF16, q_out, scales_out, stream);
}

int64_t fgs_grouped_colwise_blocks(int64_t rows, int32_t G)
{
    if (rows < 0 || G < 0) return 0;
    return rows / 128 + G;
}

int fgs_quantize_grouped_colwise(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                 const int32_t* row_index, int64_t src_rows,
                                 const int32_t* group_offsets, int32_t G,
                                 uint8_t* q, float* scales,
                                 uint8_t* qT, int64_t ldqT, float* scalesT, void* stream)
{
    if (G < 0) return fail(FGS_ERR_INVALID_ARG, "G must be >= 0");
    if (rows < 0) return fail(FGS_ERR_INVALID_ARG, "rows must be >= 0");
    int st;
    if (row_index) {
        if (src_rows < 0) return fail(FGS_ERR_INVALID_ARG, "src_rows must be >= 0");
        st = check_bf16_source(x, src_rows, cols, ldx);
    } else {
        st = check_bf16_source(x, rows, cols, ldx);
    }
    if (st != FGS_OK) return st;
    if (rows == 0 || cols == 0 || G == 0 || (!q && !qT)) return ok();
    if (!group_offsets) return fail(FGS_ERR_INVALID_ARG, "group_offsets is NULL");
    if (row_index && src_rows > 0 && !x) return fail(FGS_ERR_INVALID_ARG, "x is NULL");
    if (qT && !scalesT) return fail(FGS_ERR_INVALID_ARG, "scalesT is NULL while qT is given");
    const int64_t blocks = fgs_grouped_colwise_blocks(rows, G);
    if (blocks > kMaxRowBlocks)
        return fail(FGS_ERR_UNSUPPORTED, "rows / 128 + G = %lld token blocks (at most %lld)", (long long)blocks,
                    (long long)kMaxRowBlocks);
    if ((cols + 127) / 128 > kMaxColBlocks) return fail(FGS_ERR_UNSUPPORTED, "cols too large (%lld)", (long long)cols);
    if (qT) {
        if (ldqT < 128 * blocks)
            return fail(FGS_ERR_INVALID_ARG, "ldqT (%lld) < 128 * (rows / 128 + G) = %lld", (long long)ldqT,
                        (long long)(128 * blocks));
        if (ldqT % 16) return fail(FGS_ERR_UNSUPPORTED, "ldqT must be a multiple of 16");
        if (!aligned(qT, 16) || !aligned(scalesT, 4)) return fail(FGS_ERR_UNSUPPORTED, "qT must be 16-byte and scalesT 4-byte aligned");
    }
    if (q) {
        if (!scales) return fail(FGS_ERR_INVALID_ARG, "scales is NULL while q is given");
        if (cols % 128) return fail(FGS_ERR_UNSUPPORTED, "row-wise output needs cols %% 128 == 0 (cols = %lld)", (long long)cols);
        if (!aligned(q, 16) || !aligned(scales, 4)) return fail(FGS_ERR_UNSUPPORTED, "q must be 16-byte and scales 4-byte aligned");
    }
    fgs::QuantGroupedArgs a{x, rows, cols, ldx, row_index, src_rows, group_offsets, G, q, scales, qT, ldqT, scalesT};
    return hip_status(fgs::launch_quant_grouped_colwise(a, static_cast<hipStream_t>(stream)),
                      "quantize_grouped_colwise launch");
}

int fgs_swiglu_quantize_grouped(const void* gate_up, int64_t rows, int64_t inter, int64_t ld,
                                const int32_t* group_offsets, int32_t G, uint16_t* h,
                                uint8_t* q, float* scales, uint8_t* qT, int64_t ldqT, float* scalesT,
                                void* stream)
{
    if (G < 0) return fail(FGS_ERR_INVALID_ARG, "G must be >= 0");
    if (inter < 0) return fail(FGS_ERR_INVALID_ARG, "inter must be >= 0");
    int st = check_bf16_source(gate_up, rows, 2 * inter, ld);
    if (st != FGS_OK) return st;
    if (inter % 8) return fail(FGS_ERR_UNSUPPORTED, "inter must be a multiple of 8 (16-byte halves)");
    if (rows == 0 || inter == 0 || G == 0 || (!q && !qT && !h)) return ok();
    if (!group_offsets) return fail(FGS_ERR_INVALID_ARG, "group_offsets is NULL");
    if (h && !aligned(h, 16)) return fail(FGS_ERR_UNSUPPORTED, "h must be 16-byte aligned");
    if (qT && !scalesT) return fail(FGS_ERR_INVALID_ARG, "scalesT is NULL while qT is given");
    const int64_t blocks = fgs_grouped_colwise_blocks(rows, G);
    if (blocks > kMaxRowBlocks)
        return fail(FGS_ERR_UNSUPPORTED, "rows / 128 + G = %lld token blocks (at most %lld)", (long long)blocks,
                    (long long)kMaxRowBlocks);
    if ((inter + 127) / 128 > kMaxColBlocks) return fail(FGS_ERR_UNSUPPORTED, "inter too large (%lld)", (long long)inter);
    if (qT) {
        if (ldqT < 128 * blocks)
            return fail(FGS_ERR_INVALID_ARG, "ldqT (%lld) < 128 * (rows / 128 + G) = %lld", (long long)ldqT,
                        (long long)(128 * blocks));
        if (ldqT % 16) return fail(FGS_ERR_UNSUPPORTED, "ldqT must be a multiple of 16");
        if (!aligned(qT, 16) || !aligned(scalesT, 4)) return fail(FGS_ERR_UNSUPPORTED, "qT must be 16-byte and scalesT 4-byte aligned");
    }
    if (q) {
        if (!scales) return fail(FGS_ERR_INVALID_ARG, "scales is NULL while q is given");
        if (inter % 128) return fail(FGS_ERR_UNSUPPORTED, "row-wise output needs inter %% 128 == 0 (inter = %lld)", (long long)inter);
        if (!aligned(q, 16) || !aligned(scales, 4)) return fail(FGS_ERR_UNSUPPORTED, "q must be 16-byte and scales 4-byte aligned");
    }
    fgs::QuantGroupedArgs a{gate_up, rows, inter, ld, nullptr, 0, group_offsets, G, q, scales, qT, ldqT, scalesT, 1, h};
    return hip_status(fgs::launch_quant_grouped_colwise(a, static_cast<hipStream_t>(stream)),
                      "swiglu_quantize_grouped launch");
}

static int wgrad_impl(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets,
                      int32_t G, int64_t total_T, int64_t M, int64_t N,
                      void* C, int64_t ldc, int out_dtype, void* stream, bool fp8_mma)
{
    if (G < 0) return fail(FGS_ERR_INVALID_ARG, "G must be >= 0");
    if (total_T < 0) return fail(FGS_ERR_INVALID_ARG, "total_T must be >= 0");
    if (G == 0) {
        if (M < 0 || N < 0) return fail(FGS_ERR_INVALID_ARG, "M, N, K must be >= 0");
        return ok();
    }
    const int64_t Kcap = 128 * fgs_grouped_colwise_blocks(total_T, G);
    int st = check_gemm_common(A, B, M, N, Kcap, C, ldc, out_dtype);
    if (st != FGS_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!group_offsets) return fail(FGS_ERR_INVALID_ARG, "group_offsets is NULL");
    if (A->elem != FGS_ELEM_E4M3 || A->scale_mode != FGS_SCALE_TILE_1x128 || B->scale_mode != FGS_SCALE_TILE_1x128)
        return fail(FGS_ERR_UNSUPPORTED, "grouped wgrad supports E4M3 TILE_1x128 x TILE_1x128");
    if (M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30)) return fail(FGS_ERR_UNSUPPORTED, "sizes too large");
    const int64_t tiles = (int64_t)G * ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > 0x7FFFFFFF) return fail(FGS_ERR_UNSUPPORTED, "too many tiles");
    fgs::GemmArgs a{*A, *B, M, N, Kcap, C, ldc, out_dtype == FGS_OUT_BF16, group_offsets, G, 1, total_T,
                    nullptr, nullptr, fp8_mma ? 1 : 0, FGS_TILE_AUTO};
    return hip_status(fgs::launch_gemm_fp8(a, static_cast<hipStream_t>(stream)), "grouped_wgrad_block_scaled launch");
}

int fgs_grouped_wgrad_block_scaled(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets,
                                   int32_t G, int64_t total_T, int64_t M, int64_t N,
                                   void* C, int64_t ldc, int out_dtype, void* stream)
{
    return wgrad_impl(A, B, group_offsets, G, total_T, M, N, C, ldc, out_dtype, stream, false);
}

int fgs_grouped_wgrad_block_scaled_fp8mma(const fgs_operand* A, const fgs_operand* B, const int32_t* group_offsets,
                                          int32_t G, int64_t total_T, int64_t M, int64_t N,
                                          void* C, int64_t ldc, int out_dtype, void* stream)
{
    return wgrad_impl(A, B, group_offsets, G, total_T, M, N, C, ldc, out_dtype, stream, true);
}

} // extern "C"
