/*
 * fgs.h -- C ABI of libfgs: fine-grained scaled low-precision quantization
 * and block-scaled GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operations follow three web pages on fine-grained scaled training:
 *  [DSV3]  "Can you explain the role of FP8 precision in DeepSeek-V3
 *          training" (codingmall.com): "Mixed precision framework" (GEMMs in
 *          FP8), "Fine-grained quantization" (activations in 1x128 tiles,
 *          weights in 128x128 blocks, each scaled independently), "Online
 *          quantization" (scales from the current tile/block, no history),
 *          "Increasing accumulation precision" (partial sums promoted to
 *          FP32 registers at intervals), "Unified E4M3 format" (E4M3 in the
 *          forward and backward passes).
 *  [NEMO]  "Accelerating FP8 training performance with the NVIDIA NeMo
 *          framework" (hyper.ai): per-tensor and block-wise scaling recipes,
 *          MXFP8 with one scale per block of 32 values.
 *  [NVFP4] "NVIDIA developed a method to train neural networks at 4-bit"
 *          (news.hamidun.com), "How it works": the 4-bit NVFP4 format, random
 *          16x16 Hadamard transforms of gradient inputs, stochastic rounding.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL = the null stream) and the call returns at once.
 *  - Matrices are row-major.  BF16 inputs are raw 16-bit patterns.  Every
 *    GEMM operand is K-contiguous ("NT"): C[m][n] = sum_k A[m][k] * B[n][k].
 *  - Element codes: E4M3 = OCP E4M3FN byte (0x7E = 448, 0x7F/0xFF NaN);
 *    E5M2 = OCP E5M2 byte (0x7B = 57344); E2M1 = OCP FP4 nibble, two per
 *    byte, element 2j in the low nibble.
 *  - Quantization is online: every scale comes from the amax of the data
 *    being quantized in this call (except fgs_quantize_delayed, whose scale
 *    comes from an amax history).  FP32-scaled blocks use
 *    scale = fl32(amax / 448) and code = E4M3_RNE_SAT(fl32(x / scale));
 *    an all-zero block gets scale 1 and signed-zero codes; a block holding
 *    NaN/Inf gets scale NaN and NaN codes.
 *  - Status: FGS_OK, or a negative fgs_status.  Argument errors are detected
 *    before any HIP call and leave outputs untouched; fgs_last_error() then
 *    returns a message (thread-local).  A kernel launch failure returns
 *    FGS_ERR_HIP; a fault inside a kernel surfaces at the caller's next
 *    synchronisation.
 *  - Pointers must be 16-byte aligned; row strides are in elements.  GEMM
 *    operand row strides must stay below 2^24 bytes.
 *  - GEMMs sum exact products in FP32 (the codes are decoded exactly to
 *    FP16/BF16 for the matrix unit), except the *_fp8mma entry points,
 *    which use the FP8 matrix instructions and a looser error bound.
 */
#ifndef FGS_H
#define FGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FGS_OK = 0,
    FGS_ERR_INVALID_ARG = -1,
    FGS_ERR_UNSUPPORTED = -2,
    FGS_ERR_HIP = -3
} fgs_status;

/* Element formats of a quantized operand. */
typedef enum {
    FGS_ELEM_E4M3 = 0, /* one byte per element */
    FGS_ELEM_E2M1 = 1, /* two elements per byte */
    FGS_ELEM_E5M2 = 2  /* one byte per element: OCP E5M2 (bias 15, 0x7B =
                          57344, 0x7C Inf, 0x7D-0x7F NaN); TENSOR scale only */
} fgs_elem;

/*
 * Scale granularities.  For an operand of R rows and contraction length K
 * (K-contiguous codes, row stride ld):
 *  FGS_SCALE_TENSOR        FP32 [1]                     [NEMO] per-tensor
 *  FGS_SCALE_TILE_1x128    FP32 [K/128][R]  (tile-column-major, so one
 *                          K-block's scales are contiguous)  [DSV3] 1x128
 *  FGS_SCALE_BLOCK_128x128 FP32 [ceil(R/128)][K/128]         [DSV3] 128x128
 *  FGS_SCALE_MX32_E8M0     u8   [R][K/32]  2^(c-127)          [NEMO] MXFP8
 *  FGS_SCALE_NV16_E4M3     u8   [R][K/16]  E4M3 codes, times an FP32 tensor
 *                          scale                              [NVFP4]
 */
typedef enum {
    FGS_SCALE_TENSOR = 0,
    FGS_SCALE_TILE_1x128 = 1,
    FGS_SCALE_BLOCK_128x128 = 2,
    FGS_SCALE_MX32_E8M0 = 3,
    FGS_SCALE_NV16_E4M3 = 4
} fgs_scale;

typedef enum { FGS_ROUND_RNE = 0, FGS_ROUND_STOCHASTIC = 1 } fgs_round;
typedef enum { FGS_OUT_FP32 = 0, FGS_OUT_BF16 = 1 } fgs_out;

/* One quantized GEMM operand: R rows x K, K-contiguous. */
typedef struct {
    const void *data;          /* codes (device)                                  */
    int64_t ld;                /* row stride in ELEMENTS (E2M1: elements, even)   */
    int32_t elem;              /* fgs_elem                                        */
    int32_t scale_mode;        /* fgs_scale                                       */
    const void *scales;        /* device; layout per fgs_scale                    */
    const float *tensor_scale; /* device FP32 [1]; NV16 only, else NULL           */
} fgs_operand;

/*
 * fgs_quantize_blockwise -- online FP32-scaled E4M3 quantization.
 *   [DSV3] "Fine-grained quantization", "Online quantization";
 *   [NEMO] per-tensor current scaling.
 * x        BF16 [rows x cols], row stride ldx (elements, multiple of 8).
 * mode     FGS_SCALE_TILE_1x128 | FGS_SCALE_BLOCK_128x128 | FGS_SCALE_TENSOR.
 * Row-wise output (quantized along cols; NULL q skips it; needs cols % 128 == 0):
 *   q       E4M3 [rows x cols] (dense), scales per mode for R = rows, K = cols.
 * Column-wise output (the transpose, quantized along rows; NULL qT skips it;
 *   needs rows % 128 == 0):
 *   qT      E4M3 [cols x rows] (dense), scalesT per mode for R = cols, K = rows.
 *   TILE re-quantizes each 128-row column segment from the BF16 source
 *   (the wgrad operand); BLOCK and TENSOR transpose the row-wise codes and
 *   scale grid (the 128x128 grid and a single scale are transpose-invariant).
 * Both outputs come from one read of x.  TENSOR mode needs a device
 *   workspace (4-byte aligned, at least 4 bytes; its contents are scratch):
 *   the amax pass stores one 4-byte partial per workgroup and the cast pass
 *   takes their max.  fgs_workspace_bytes() bytes let it run two amax
 *   workgroups per compute unit; a smaller workspace runs fewer (same
 *   result).  TILE/BLOCK ignore it.
 * rows and cols may be 0 (nothing is enqueued).
 */
int fgs_quantize_blockwise(const void *x, int64_t rows, int64_t cols, int64_t ldx,
                           int mode, uint8_t *q, float *scales,
                           uint8_t *qT, float *scalesT,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * fgs_quantize_blockwise_noalloc -- fgs_quantize_blockwise without a
 *   workspace argument, for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid allocation).  It calls no allocator: TENSOR mode keeps its amax
 *   partials in the library's own device scratch, a fixed 4 KiB array per
 *   GPU (1024 four-byte slots) that each GPU holds until the process ends.
 *   The amax pass runs at most one workgroup per slot whatever the input
 *   size, so no input is too large for it.  The first call on a device
 *   resolves that array's address on the device (a HIP call, after the
 *   argument checks); a failure there returns FGS_ERR_HIP.
 * Arguments, layouts, results, ownership and errors as fgs_quantize_blockwise
 *   (the results are bit-identical).  Every slot a call reads is written by
 *   the same call first, so nothing carried over from an earlier call
 *   matters; but calls that overlap on one GPU (on different streams, or
 *   from different threads) share the array and race: the caller orders
 *   them.  TILE and BLOCK modes use no scratch.
 */
int fgs_quantize_blockwise_noalloc(const void *x, int64_t rows, int64_t cols, int64_t ldx,
                                   int mode, uint8_t *q, float *scales,
                                   uint8_t *qT, float *scalesT, void *stream);

/*
 * fgs_quantize_delayed -- per-tensor DELAYED scaling to E4M3 or E5M2: the
 *   scale comes from the amaxes of earlier steps, the recipe that online
 *   scaling replaces, and E5M2 gives the hybrid recipe (E4M3 forward, E5M2
 *   gradients) that the single E4M3 format replaces.   [DSV3] "Online
 *   quantization", "Unified E4M3 format".
 * elem     FGS_ELEM_E4M3 (fmax 448) or FGS_ELEM_E5M2 (fmax 57344).
 * amax_history  DEVICE FP32 [history_len] (1 <= history_len <= 65536),
 *   owned by the caller, all zeros before the first step.  The call reads
 *   every entry: hmax = NaN-propagating max of |entries|; scale s = 1 if
 *   hmax == 0, NaN if hmax is not finite, else fl32(hmax / fmax).  Then it
 *   stores this tensor's amax (NaN-propagating max |x|) into
 *   amax_history[slot] (0 <= slot < history_len; a rolling window passes
 *   slot = step % history_len).  rows or cols 0 record 0.
 * code = ENC_RNE_SAT(fl32(x / s)): RNE to the nearest code, ties to even,
 *   |x / s| beyond fmax (and +-Inf) saturating to +-fmax, the sign kept
 *   (-0 -> 0x80), NaN (or a NaN scale) -> 0x7F.
 * One read of x (the scale is known before the data).
 * Row-wise (NULL q skips it): q [rows x cols].  Column-wise (NULL qT skips
 *   it; needs rows % 128 == 0): qT [cols x rows], the byte transpose (one
 *   scale is transpose-invariant).  scale: DEVICE FP32 [1], the s used (both
 *   outputs' FGS_SCALE_TENSOR scale).
 */
int fgs_quantize_delayed(const void *x, int64_t rows, int64_t cols, int64_t ldx, int elem,
                         float *amax_history, int32_t history_len, int32_t slot,
                         uint8_t *q, uint8_t *qT, float *scale, void *stream);

/*
 * fgs_quantize_mx -- MXFP8: E4M3 codes with one E8M0 scale 2^e per 32
 *   contiguous elements, e the smallest integer with amax <= 448 * 2^e
 *   (clamped to [-127, 127]); code = E4M3_RNE_SAT(x * 2^-e).   [NEMO] MXFP8.
 * Row-wise (needs cols % 32 == 0): q [rows x cols], scales u8 [rows][cols/32].
 * Column-wise (needs rows % 128 == 0): qT [cols x rows], scalesT u8
 *   [cols][rows/32] (blocks of 32 along the source rows).
 */
int fgs_quantize_mx(const void *x, int64_t rows, int64_t cols, int64_t ldx,
                    uint8_t *q, uint8_t *scales, uint8_t *qT, uint8_t *scalesT,
                    void *stream);

/*
 * fgs_quantize_nvfp4 -- NVFP4: E2M1 codes, one E4M3 scale per 16 contiguous
 *   elements, one FP32 tensor scale per output.   [NVFP4] "How it works".
 *   s_t = fl32(amax_t / 2688); s_b = E4M3(fl32(amax_b / fl32(6 s_t)));
 *   code = E2M1(sat6(fl32(x / fl32(dec(s_b) * s_t)))), RNE or stochastic.
 * rht_mask bit 0: apply the random 16x16 Hadamard transform (signs from
 *   rht_seed) along the quantized dimension of the row-wise output; bit 1:
 *   same for the column-wise output.  The transform precedes the amax.
 * round    FGS_ROUND_RNE or FGS_ROUND_STOCHASTIC (applies to both outputs);
 *   the SR word r of an element hashes sr_seed with its linear index
 *   row * cols + col in x, and |y| between neighbours lo < hi rounds up iff
 *   (r >> 10) < floor(p * 2^22), p = (|y| - lo) / (hi - lo): the stochastic
 *   rounding is resolved to 22 bits.
 * Row-wise (needs cols % 16 == 0): q [rows x cols/2], scales u8 [rows][cols/16].
 * Column-wise (needs rows % 128 == 0): qT [cols x rows/2], scalesT u8
 *   [cols][rows/16].
 * tensor_scale  device FP32 [2]: [0] row-wise s_t, [1] column-wise s_t.
 * workspace     device scratch, 4-byte aligned, at least 8 bytes: two 4-byte
 *               amax partials per amax workgroup (fgs_workspace_bytes()
 *               bytes give two workgroups per compute unit; fewer bytes,
 *               fewer workgroups, same result).
 */
int fgs_quantize_nvfp4(const void *x, int64_t rows, int64_t cols, int64_t ldx,
                       int rht_mask, uint64_t rht_seed, int round, uint64_t sr_seed,
                       uint8_t *q, uint8_t *scales, uint8_t *qT, uint8_t *scalesT,
                       float *tensor_scale, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * fgs_gemm_block_scaled -- C[M x N] = sum_k A^[m,k] * B^[n,k] with scaled
 *   low-precision operands.   [DSV3] "Mixed precision framework",
 *   "Increasing accumulation precision"; [NEMO]; [NVFP4].
 * A: M x K operand, B: N x K operand (fgs_operand).  Supported pairs:
 *   E4M3 with A in {TILE_1x128, TENSOR} and B in {BLOCK_128x128, TILE_1x128,
 *     TENSOR}: MFMA partial sums over one 128-deep K block are scaled by
 *     sA * sB and added into FP32 accumulators once per block (promotion);
 *   E4M3 with MX32_E8M0 on both: each code decoded exactly to BF16 as
 *     code * 2^(e - E) (E the largest non-NaN scale exponent of the row (A)
 *     or of the workgroup tile's rows (B) over all of K), BF16 MFMA with
 *     FP32 accumulation over all of K, then 2^(E_A + E_B) applied by
 *     exponent arithmetic; exact while every pair of meeting blocks has
 *     (e_A - E_A) + (e_B - E_B) >= -108 (each decoded code a BF16 number,
 *     each product a normal FP32 number); a pair further apart adds less
 *     than 2^-90 * 2^(E_A + E_B - 254) per product; a NaN scale byte makes
 *     its A row or B column of C NaN;
 *   E4M3 or E5M2 on each side with TENSOR on both (the delayed-scaling
 *     recipes; E5M2 gradients against E4M3 weights or activations): every
 *     E5M2 code is exactly the FP16 number with the code as its upper byte,
 *     FP16 MFMA with FP32 accumulation over all of K, sA * sB at the end;
 *   E2M1 with NV16_E4M3 on both: each code times its E4M3 block scale,
 *     exact in FP16, FP16 MFMA with FP32 accumulation over all of K, the
 *     two tensor scales applied at the end.
 * The products of the decoded operands are exact and the sums are FP32
 * (the matrix unit's own FP8 path rounds inside each group of 8 products,
 * which the bound below does not allow).
 * K must be a positive multiple of 128 (K = 0 with M, N > 0 returns
 *   FGS_ERR_UNSUPPORTED); M, N >= 0 arbitrary, and M or N = 0 launches nothing.
 * C: FP32 or BF16 (RNE) [M x N], row stride ldc >= N (elements).
 * Accuracy: |C - C_ref| <= 1e-5 * sum_k |a_k b_k| + 1e-6 for FP32 output,
 * C_ref the exact product of the dequantized operands.
 * The caller guarantees that code and scale buffers hold what the layouts
 * above require for M, N, K (the library cannot see buffer sizes).
 */
int fgs_gemm_block_scaled(const fgs_operand *A, const fgs_operand *B,
                          int64_t M, int64_t N, int64_t K,
                          void *C, int64_t ldc, int out_dtype, void *stream);

/*
 * fgs_gemm_block_scaled_fp8mma -- the same product on the FP8 matrix
 *   instructions, as the pages' own design does it: the FP8 codes go to the
 *   matrix unit as they are, its partial sums over each 128-deep K block are
 *   promoted into FP32 accumulators with sA * sB (1x128 / 128x128 scales),
 *   and MX E8M0 scales are applied by the scaled instruction itself.
 *   [DSV3] "Increasing accumulation precision" (limited accumulation inside
 *   the matrix unit, promotion to FP32 at a fixed interval); [NEMO] MXFP8.
 * Arguments, layouts, ownership and errors as fgs_gemm_block_scaled, for
 *   the E4M3 / E5M2 operand pairs it lists (FP32-scaled and MX32_E8M0);
 *   E2M1 operands return FGS_ERR_UNSUPPORTED.
 * Accuracy: the instruction adds each group of 8 consecutive products with
 *   about 13 bits below the largest of them, an error of at most
 *   2^-10 * sum |a_k b_k| per group; with the FP32 sums that follow,
 *   |C - C_ref| <= 2^-9 * sum_k |a_k b_k| + 1e-6 for K <= 65536 (FP32
 *   output; BF16 output adds one BF16 ulp).  This is looser than the 1e-5
 *   bound of fgs_gemm_block_scaled, which stays the exact default.
 * MX: a scale byte of 0xFF (NaN) is passed to the instruction unchanged;
 *   products whose scales leave the FP32 range overflow or underflow as the
 *   instruction does (the default GEMM rescales them exactly).
 */
int fgs_gemm_block_scaled_fp8mma(const fgs_operand *A, const fgs_operand *B,
                                 int64_t M, int64_t N, int64_t K,
                                 void *C, int64_t ldc, int out_dtype, void *stream);

/*
 * fgs_grouped_gemm_block_scaled -- MoE expert GEMMs: for each group g,
 *   rows group_offsets[g] .. group_offsets[g+1]-1 of A times B_g^T.
 *   [DSV3] "Mixed precision framework" (expert GEMMs in FP8, gating kept in
 *   higher precision and outside this call).
 * A: total_M x K, E4M3 TILE_1x128 (scales [K/128][total_M]).
 * B: G x N x K E4M3 codes (group g at g*N*ld), BLOCK_128x128 scales
 *   [G][ceil(N/128)][K/128] (group g at g*ceil(N/128)*(K/128)).
 * group_offsets: DEVICE int32 [G+1], non-decreasing, offsets[0] = 0,
 *   offsets[G] = total_M.  Read on the device (no host synchronisation);
 *   offsets outside [0, total_M] make the affected groups write nothing.
 * C: [total_M x N] FP32 or BF16.  Rows not covered by any group are not written.
 */
int fgs_grouped_gemm_block_scaled(const fgs_operand *A, const fgs_operand *B,
                                  const int32_t *group_offsets, int32_t G,
                                  int64_t total_M, int64_t N, int64_t K,
                                  void *C, int64_t ldc, int out_dtype, void *stream);

/*
 * fgs_grouped_gemm_block_scaled_fp8mma -- the grouped (MoE) GEMM above on
 *   the FP8 matrix instructions, promoted to FP32 once per 128-deep K block,
 *   for callers who accept that accumulation (see
 *   fgs_gemm_block_scaled_fp8mma).   [DSV3] "Increasing accumulation
 *   precision".  Arguments, layouts, ownership and errors as
 *   fgs_grouped_gemm_block_scaled.  Accuracy: |C - C_ref| <= 2^-9 *
 *   sum_k |a_k b_k| + 1e-6 per group (FP32 output; BF16 adds one BF16 ulp).
 */
int fgs_grouped_gemm_block_scaled_fp8mma(const fgs_operand *A, const fgs_operand *B,
                                         const int32_t *group_offsets, int32_t G,
                                         int64_t total_M, int64_t N, int64_t K,
                                         void *C, int64_t ldc, int out_dtype, void *stream);

/*
 * fgs_quantize_grouped_colwise -- the MoE weight-gradient operands: per-group
 *   transposed 1x128 E4M3 quantization.   [DSV3] "Fine-grained
 *   quantization", "Online quantization", "Mixed precision framework" (the
 *   expert GEMMs, wgrad included, in FP8 with 1x128 tiles along the
 *   contraction, which for wgrad runs over each expert's tokens).
 * x        BF16 [rows x cols] (or [src_rows x cols] with row_index), row
 *          stride ldx (elements, multiple of 8); row t is a token, grouped by
 *          expert.
 * row_index  NULL, or DEVICE int32 [rows]: the MoE dispatch gather fused
 *          into the read.  Row t of the matrix the groups index is then row
 *          row_index[t] of x (x has src_rows rows; an index outside
 *          [0, src_rows) reads as a row of zeros), so the permuted BF16 copy is
 *          never written.  Everything below refers to the gathered rows.
 *          [DSV3] "Mixed precision framework" (expert GEMMs in FP8).
 * group_offsets  DEVICE int32 [G+1]: group g is rows offsets[g] ..
 *          offsets[g+1]-1 (M_g tokens).  Read on the device.  A group with
 *          offsets[g] < 0, offsets[g+1] < offsets[g] or offsets[g+1] > rows
 *          is treated as empty; offsets that decrease from one group to the
 *          next give unspecified codes, but every write stays inside the
 *          buffers below.
 * Column-wise output (NULL qT skips it): group g's transpose [cols x M_g] in 1x128
 *   tiles along its tokens (a tile never holds two groups' tokens; the last
 *   one is partial when M_g % 128 != 0, scaled from the tokens present and
 *   padded with code 0x00, or 0x7F like the rest of a tile whose scale is
 *   NaN).  Group g occupies the 128-column blocks
 *   kb_g .. kb_g + ceil(M_g/128) - 1 with kb_g = floor(offsets[g]/128) + g,
 *   so the layout needs no scan and no host synchronisation; blocks no group
 *   owns are not written.  There are at most
 *   fgs_grouped_colwise_blocks(rows, G) = floor(rows/128) + G blocks; more
 *   than 65535 returns FGS_ERR_UNSUPPORTED.
 *   qT       E4M3 [cols x ldqT], ldqT >= 128 * fgs_grouped_colwise_blocks,
 *            ldqT % 16 == 0.
 *   scalesT  FP32 [fgs_grouped_colwise_blocks][cols] (the TILE_1x128 layout
 *            of an operand of cols rows and K = 128 * blocks).
 * Row-wise output (NULL q skips it; needs cols % 128 == 0): the ordinary
 *   1x128 quantization of every row that a valid group covers, from the same
 *   read: q [rows x cols], scales [cols/128][rows]; rows of no group are not
 *   written.  With neither output nothing is enqueued.
 */
int fgs_quantize_grouped_colwise(const void *x, int64_t rows, int64_t cols, int64_t ldx,
                                 const int32_t *row_index, int64_t src_rows,
                                 const int32_t *group_offsets, int32_t G,
                                 uint8_t *q, float *scales,
                                 uint8_t *qT, int64_t ldqT, float *scalesT, void *stream);

/*
 * fgs_swiglu_quantize_grouped -- the SwiGLU activation between the two
 *   expert GEMMs fused into the grouped quantizer of the down projection's
 *   operands, so the activation is never written and read back in BF16.
 *   [DSV3] "Mixed precision framework" (the expert GEMMs run in FP8); the
 *   activation itself is not on the pages: SwiGLU is the DeepSeek-V3
 *   expert's, computed here in FP32 before the FP8 cast.
 * gate_up  BF16 [rows x 2*inter], row stride ld (multiple of 8; inter a
 *          multiple of 8): the gate/up GEMM output, gate = columns
 *          0..inter-1, up = columns inter..2*inter-1.
 * The quantized matrix is h [rows x inter] with
 *   h = BF16_RNE(fl32(fl32(g * sig) * u)), sig = 1 / (1 + e) for g >= 0 and
 *   e / (1 + e) for g < 0, e = expf(-|g|), everything in FP32 (expf to
 *   within a few ulp), so h is within one BF16 ulp of the exact SwiGLU; the
 *   codes are exactly the 1x128 quantization of that h.
 * h (optional, NULL skips it): BF16 [rows x inter] of the rows a valid group
 *   covers (for a backward pass that wants it).
 * group_offsets, G, q / scales, qT / ldqT / scalesT: as for
 *   fgs_quantize_grouped_colwise with cols = inter (no gather).
 */
int fgs_swiglu_quantize_grouped(const void *gate_up, int64_t rows, int64_t inter, int64_t ld,
                                const int32_t *group_offsets, int32_t G, uint16_t *h,
                                uint8_t *q, float *scales, uint8_t *qT, int64_t ldqT, float *scalesT,
                                void *stream);

/* Number of 128-token blocks of the per-group column-wise layout for rows
 * tokens in G groups: floor(rows/128) + G (0 for negative arguments). */
int64_t fgs_grouped_colwise_blocks(int64_t rows, int32_t G);

/*
 * fgs_grouped_wgrad_block_scaled -- MoE expert weight gradients: for every
 *   group g, C_g[m][n] = sum over the tokens t of group g of A^[m,t] B^[n,t].
 *   [DSV3] "Mixed precision framework", "Fine-grained quantization",
 *   "Increasing accumulation precision" (partial sums over each 128-token
 *   tile scaled by both tiles' scales and added into FP32 accumulators).
 * A: M x (128 * blocks) E4M3 TILE_1x128 operand from
 *   fgs_quantize_grouped_colwise of dY [total_T x M] (ld = its ldqT).
 * B: N x (128 * blocks) E4M3 TILE_1x128 operand, the same for X [total_T x N].
 *   blocks = fgs_grouped_colwise_blocks(total_T, G).
 * group_offsets: the DEVICE int32 [G+1] both operands were quantized with.
 * C: G matrices [M x N] of FP32 or BF16 (RNE), C_g at C + g * M * ldc,
 *   row stride ldc >= N.  A group without tokens (or one the quantizer
 *   treats as empty) gets C_g = 0.
 * Accuracy as fgs_gemm_block_scaled.
 */
int fgs_grouped_wgrad_block_scaled(const fgs_operand *A, const fgs_operand *B,
                                   const int32_t *group_offsets, int32_t G, int64_t total_T,
                                   int64_t M, int64_t N, void *C, int64_t ldc, int out_dtype,
                                   void *stream);

/*
 * fgs_grouped_wgrad_block_scaled_fp8mma -- the per-expert weight gradient
 *   above on the FP8 matrix instructions, promoted to FP32 once per
 *   128-token block.   [DSV3] "Increasing accumulation precision".
 *   Arguments, layouts, ownership and errors as
 *   fgs_grouped_wgrad_block_scaled.  Accuracy: |dW_g - ref| <= 2^-9 *
 *   sum_t |a_t b_t| + 1e-6 (FP32 output; BF16 adds one BF16 ulp).
 */
int fgs_grouped_wgrad_block_scaled_fp8mma(const fgs_operand *A, const fgs_operand *B,
                                          const int32_t *group_offsets, int32_t G, int64_t total_T,
                                          int64_t M, int64_t N, void *C, int64_t ldc, int out_dtype,
                                          void *stream);

/*
 * fgs_gemm_block_scaled_fp8out / fgs_grouped_gemm_block_scaled_fp8out --
 *   the GEMMs above with BF16 output, whose epilogue also quantizes that BF16
 *   output in 1x128 tiles along N for the next layer: the next GEMM's A
 *   operand without a BF16 round trip.   [DSV3] "Fine-grained
 *   quantization", "Online quantization" (the same rule as
 *   fgs_quantize_blockwise's row-wise TILE_1x128 output, applied to the
 *   BF16-rounded C).
 * C may be NULL (no BF16 output; ldc is then ignored).
 * q_out      E4M3 [M x N] (dense, 4-byte aligned); scales_out FP32
 *            [N/128][M] (the TILE_1x128 layout for R = M, K = N).  The
 *            grouped form writes the rows its groups cover.
 * Needs N % 128 == 0.  Other arguments and supported operands as for the
 * BF16-output GEMMs.
 */
int fgs_gemm_block_scaled_fp8out(const fgs_operand *A, const fgs_operand *B,
                                 int64_t M, int64_t N, int64_t K, void *C, int64_t ldc,
                                 uint8_t *q_out, float *scales_out, void *stream);
int fgs_grouped_gemm_block_scaled_fp8out(const fgs_operand *A, const fgs_operand *B,
                                         const int32_t *group_offsets, int32_t G,
                                         int64_t total_M, int64_t N, int64_t K, void *C, int64_t ldc,
                                         uint8_t *q_out, float *scales_out, void *stream);

/*
 * fgs_gemm_block_scaled_ex -- fgs_gemm_block_scaled with per-call options:
 *   the workgroup tile, the matrix instructions, and the E4M3-output
 *   epilogue.   [DSV3] "Mixed precision framework", "Increasing
 *   accumulation precision"; [NEMO]; [NVFP4].
 * opts     NULL, or a caller-owned host struct read during the call only.
 *          NULL and an all-zero struct both mean: automatic tile, exact
 *          path, no E4M3 output, i.e. fgs_gemm_block_scaled.
 *   tile        FGS_TILE_AUTO picks the workgroup tile per problem from the
 *               tile counts and the device's compute units; FGS_TILE_NARROW
 *               forces 256 x 128 outputs per workgroup, FGS_TILE_WIDE
 *               256 x 256.  Only the speed and the order of the FP32 sums
 *               inside one 128-deep block differ: per-tensor E4M3/E5M2 and
 *               NVFP4 results are bit-identical across tiles, and every mode
 *               meets the accuracy bound on either tile.
 *   fp8_mma     0: exact (codes decoded to FP16/BF16); 1: the FP8 matrix
 *               instructions, as fgs_gemm_block_scaled_fp8mma (with its
 *               looser bound).
 *   q_out, scales_out  both NULL, or the E4M3-output epilogue of
 *               fgs_gemm_block_scaled_fp8out (then out_dtype must be
 *               FGS_OUT_BF16, C may be NULL, N % 128 == 0, and fp8_mma must
 *               be 0).
 *   workspace, workspace_bytes  NULL / 0, or DEVICE scratch (16-byte
 *               aligned, owned by the caller, not read before it is
 *               written) of at least fgs_gemm_workspace_bytes(A->scale_mode,
 *               M, N) bytes.  MXFP8 on the exact path then forms each row's
 *               largest scale exponent once, in a pass of its own enqueued
 *               before the GEMM; without it every workgroup tile scans the
 *               scale bytes of its own rows (slower: on the Llama-3.1-405B
 *               MXFP8 layers, about 3% of the GEMM time more).  The results
 *               are the same bits either way.  Other modes ignore it.  A
 *               workspace given with fewer bytes than required, or
 *               misaligned, returns FGS_ERR_INVALID_ARG.
 * Other arguments, layouts, ownership and errors as fgs_gemm_block_scaled;
 * an unknown tile or fp8_mma value returns FGS_ERR_INVALID_ARG.  The library
 * keeps no state between calls: every choice is made from the arguments.
 */
enum { FGS_TILE_AUTO = 0, FGS_TILE_NARROW = 1, FGS_TILE_WIDE = 2 };
typedef struct {
    int32_t tile;          /* FGS_TILE_*                                      */
    int32_t fp8_mma;       /* 0 or 1                                          */
    uint8_t *q_out;        /* device E4M3 [M x N] or NULL                     */
    float *scales_out;     /* device FP32 [N/128][M] or NULL                  */
    void *workspace;       /* device scratch or NULL                          */
    size_t workspace_bytes;
} fgs_gemm_options;
int fgs_gemm_block_scaled_ex(const fgs_operand *A, const fgs_operand *B,
                             int64_t M, int64_t N, int64_t K, void *C, int64_t ldc,
                             int out_dtype, const fgs_gemm_options *opts, void *stream);

/*
 * fgs_gemm_kernel_name -- the kernel instantiation that
 *   fgs_gemm_block_scaled_ex(A, B, M, N, K, C, ldc, out_dtype, opts, ...)
 *   would launch, named as profilers print it (without namespaces and
 *   arguments, e.g. "gemm_block_scaled_kernel<Shape<2, 4, 4>, 1, 2, true,
 *   0, 0, false>"), so timings and counters can be matched to launches.
 *   Nothing is launched and no HIP call is made beyond reading the current
 *   device's compute-unit count.
 * name     host buffer of len >= 2 bytes; receives a NUL-terminated string
 *          (truncated to len - 1 characters; "" when M or N is 0).
 * Returns what the GEMM call would return for these operands, shapes and
 * options (an argument error leaves name empty).
 */
int fgs_gemm_kernel_name(const fgs_operand *A, const fgs_operand *B, int64_t M, int64_t N, int64_t K,
                         int out_dtype, const fgs_gemm_options *opts, char *name, size_t len);

/* Device workspace needed by TENSOR-mode and NVFP4 quantization (bytes). */
size_t fgs_workspace_bytes(int64_t rows, int64_t cols);

/* Device workspace the GEMM options can bring for an M x N product whose A
 * operand has scale mode a_scale_mode: 2 (M + N) bytes for
 * FGS_SCALE_MX32_E8M0 (one reference byte and one NaN flag per row of A and
 * of B), 0 for the other modes and for negative sizes. */
size_t fgs_gemm_workspace_bytes(int a_scale_mode, int64_t M, int64_t N);

/* Message for the last error on this thread ("" if none); never NULL. */
const char *fgs_last_error(void);

/* Library version string. */
const char *fgs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FGS_H */
