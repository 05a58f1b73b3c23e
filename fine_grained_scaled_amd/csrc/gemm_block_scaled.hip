// gemm_block_scaled.hip -- the block-scaled low-precision GEMM on gfx950:
// FP32-scaled E4M3 (1x128 / 128x128 / per-tensor), MXFP8 and NVFP4 operands,
// and the grouped (MoE) variant of the E4M3 blockwise case.
//
// "Can you explain the role of FP8 precision in DeepSeek-V3 training":
// section "Mixed precision framework" (the GEMMs run on FP8 operands),
// "Fine-grained quantization" (1x128 activation tiles x 128x128 weight
// blocks) and "Increasing accumulation precision" (the matrix unit's own
// accumulation is limited, so partial sums are promoted to FP32 registers
// at fixed intervals).  Here the interval is one 128-deep K block, the scale
// block: the matrix unit forms P = sum_{k in block} qa*qb in FP32, and the
// kernel adds sA[m, kb] * sB[n, kb] * P into a separate FP32 accumulator.
// With a single per-tensor scale on both operands ("Accelerating FP8
// training performance with the NVIDIA NeMo framework", per-tensor recipe)
// no per-block factor exists: all of K accumulates in FP32 and the product
// of the two scales is applied once at the end.  MXFP8 (same page: one
// power-of-two scale per 32 values) and NVFP4 ("NVIDIA developed a method to
// train neural networks at 4-bit": E2M1 with an E4M3 scale per 16 values and
// an FP32 tensor scale) are decoded exactly into the MFMA operand format, as
// described at their decoders below.
//
// Which matrix instruction: gfx950's FP8 MFMA (v_mfma_*_f8f6f4 and the older
// *_fp8_fp8 forms) adds each group of 8 consecutive products with only about
// 13 bits below the largest of them (measured: 256 + 2^-5 survives, 256 +
// 2^-6 does not, and +x - x + tiny gives 0), the same limitation the DeepSeek
// page describes for its hardware, but *inside* one instruction, where no
// promotion interval can reach it.  Its error reaches ~1.5e-4 of
// sum_k |a_k b_k|.  The FP16 and BF16 MFMAs (v_mfma_f32_32x32x16_{f16,bf16})
// keep a full FP32-width sum (256 + 2^-15 survives).  Every E4M3 value is
// exactly an FP16 value and every product of two is exact in FP32, so the
// kernel decodes the E4M3 codes to FP16 with the hardware converter
// (v_cvt_scalef32_pk_f16_fp8, unit scale: exact for all 256 codes) and runs
// the FP16 MFMA: the result is the FP32 sum of exact products.
//
// C[m][n] = sum_k A[m][k] * B[n][k]; both operands K-contiguous.
// Workgroup: NWM x NWN waves, each owning a (32*TI) x 64 output sub-block
// (TI x 2 MFMA 32x32x16 tiles).  Promoted modes: 4 x 2 waves of 64 x 64
// (tile 256 x 128; 512 threads, two waves per SIMD so one wave's decode and
// promotion VALU work overlaps the other's MFMAs); the promoted accumulators
// and the per-block partial sums (2 x 64 VGPRs) both stay in VGPRs, which
// caps the wave tile there.  Modes without promotion (per-tensor E4M3, and
// NVFP4, whose block scales are folded into the exact decode) need no
// partial sums, so their waves can own 128 x 64 (2 x 4 waves, tile
// 256 x 256): each decoded fragment feeds more MFMAs and each staged byte
// more FLOPs; a launch takes this tile unless its last round of workgroups
// would be poorly filled (see prefer_wide).  The MoE row groups take one of
// three tiles by size (64 x 128 below 64 rows, 128 x 128 below 256, the
// 256 x 256 one above), the MoE weight gradients 2 x 2 waves of 64 x 64
// (tile 128 x 128).  K advances in
// 128-deep blocks staged in LDS as code bytes (128 bytes per row for E4M3,
// 64 for E2M1), double-buffered, by direct global->LDS loads
// (global_load_lds_dwordx4: lane i of a wave-instruction fills bytes
// 16i..16i+15 of a 1 KiB LDS span), so the next block streams in while the
// current one is multiplied without passing through registers.  The 16-byte
// chunk c of staged row r sits in LDS slot c ^ ((r >> 1) & 7) (128-byte
// rows) or c ^ ((r >> 2) & 3) (64-byte rows): the lane that fills a slot
// fetches the matching chunk, and a fragment read (16 consecutive rows, same
// chunk, 256 bytes) touches each of the 64 LDS banks once.  MFMA operands
// are swapped (B fragment first) so each lane's 16 accumulators share one
// row m: the 1x128 A scale is one value per lane and per sub-tile row.
#include <algorithm>
#include <climits>
#include <cstdio>
#include <type_traits>

#include "fgs_device.h"
#include "fgs_internal.h"

namespace fgs {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 128;      // K block: the scale block and the promotion interval

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef const __attribute__((address_space(1))) void* gbl_ptr;

// Direct global->LDS loads.  The LDS destination is the wave's span base
// (wave-uniform, passed in M0); lane i writes bytes [size*i, size*(i+1)) of it.  They are
// issued from inline assembly on purpose: seen as LDS writes, the compiler
// would make every later LDS read wait for the loads to land (it cannot tell
// that they fill the other stage of the ring), which serialises the next
// block's fetch with this block's MFMAs.  Completion is tracked by hand with
// wait_lds_dma() before the barrier that publishes a stage.  No other
// instruction of these kernels reads M0, so the statements may clobber it;
// the s_nop is the one wait state the hardware needs between an SALU write
// of M0 and an LDS-DMA load that uses it.
__device__ __forceinline__ uint32_t lds_offset(const void* p)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_ptr)p));
}
// 16 bytes per lane from a wave-uniform 64-bit base in SGPRs plus a 32-bit
// per-lane byte offset (the global instructions' saddr form), to the LDS
// address lds_addr (uniform): a K block's code loads need no per-lane
// address arithmetic, only scalar adds.
__device__ __forceinline__ void g2lds16_s(const void* sbase, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// a wave-uniform pointer, held in SGPRs
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* q)
{
    const uint64_t v = reinterpret_cast<uint64_t>(q);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void g2lds4(const void* src, void* dst_wave_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(lds_offset(dst_wave_base)) : "memory", "m0");
}
__device__ __forceinline__ void wait_lds_dma()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

struct GemmParams {
    const uint8_t* A;
    const uint8_t* B;
    const float* sA;
    const float* sB;
    const float* tsA;             // NVFP4 tensor scales (device FP32 [1])
    const float* tsB;
    const uint16_t* mx_ref;       // MXFP8 exact path: per row, A rows then B rows: reference byte | NaN flag << 8
    int64_t lda, ldb, M, N, K;    // lda, ldb in bytes
    void* C;
    int64_t ldc;
    const int32_t* offsets;
    int32_t G;
    int64_t T;                    // contraction groups: tokens (rows of the quantized source)
    int64_t b_group_stride;       // elements between groups of B codes
    int64_t sb_group_stride;      // floats between groups of B block scales
    int32_t tiles_m, tiles_n;
    uint8_t* q_out;               // BF16-out launches: 1x128 E4M3 codes of the BF16 output, or nullptr
    float* s_out;                 //   and their scales [N/128][M]
    int32_t grp_lo, grp_hi;       // row groups: this launch takes the groups of grp_lo <= rows < grp_hi
};

// FP16 x FP16 MFMA, 32x32 outputs, 16-deep K, FP32 accumulate.
__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// FP8 x FP8 MFMA, 32x32 outputs, 64-deep K, FP32 accumulate, with E8M0
// operand scales (127 = x1).  Formats (FA, FB): 0 = E4M3, 1 = E5M2.  Lane l
// holds row l % 32 and 32 codes (8 registers); both operands take the same K
// order.  The instruction's two 32-element scale blocks are bytes 0-15 of
// both lane halves (scaled by the byte of lane half 0) and bytes 16-31 of
// both halves (lane half 1's byte): measured on gfx950 with one nonzero code
// per position and distinct scales per lane half.
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

// FP8 x FP8 MFMA, 16x16 outputs, 128-deep K (one whole scale block), unit
// scales, from zero: the block's partial sums in one instruction.  Lane l
// holds row l % 16 and 32 codes of K (lane group l / 16); output lane l
// holds column l % 16 of rows 4 * (l / 16) .. +3.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int FA, int FB>
__device__ __forceinline__ f32x4 mfma8_k128(const i32x8& a, const i32x8& b)
{
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, FA, FB, 0, 127, 0, 127);
}

// FP16 x FP16 MFMA, 16x16 outputs, 32-deep K, FP32 accumulate (lane l holds
// row l % 16 and the 8 values of K of lane group l / 16).
__device__ __forceinline__ f32x4 mfma16x16(const f16x8& a, const f16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16 E4M3 codes (one 16-byte LDS read) -> two exact FP16 8-vectors: bytes
// 0..7 feed one MFMA k-step, bytes 8..15 the next.
__device__ __forceinline__ void decode16(const uint4 v, f16x8& lo, f16x8& hi)
{
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, true);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, false);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, true);
    const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.z, 1.0f, false);
    const f16x2 f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.z, 1.0f, true);
    const f16x2 g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.w, 1.0f, false);
    const f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.w, 1.0f, true);
    lo = f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    hi = f16x8{e[0], e[1], f[0], f[1], g[0], g[1], h[0], h[1]};
}

// BF16 x BF16 MFMA, 32x32 outputs, 16-deep K, FP32 accumulate.
__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 E5M2 codes -> two FP16 8-vectors (same element order as decode16).
// E5M2 is FP16 with the low 8 mantissa bits cut off, so the FP16 bits of a
// code are the code followed by a zero byte: exact for every code,
// subnormals, Inf and NaN included.
__device__ __forceinline__ void decode16_e5m2(const uint4 v, f16x8& lo, f16x8& hi)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[2 * i] = ((w[i] << 8) & 0xFF00u) | ((w[i] << 16) & 0xFF000000u);      // bytes 0, 1
        h[2 * i + 1] = ((w[i] >> 8) & 0xFF00u) | (w[i] & 0xFF000000u);          // bytes 2, 3
    }
    lo = __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
    hi = __builtin_bit_cast(f16x8, make_uint4(h[4], h[5], h[6], h[7]));
}

// One operand's 8 byte codes (E4M3, or E5M2 when E5) -> FP16: the lower
// (or upper) half of what decode16 / decode16_e5m2 return for 16 codes.
template <bool E5>
__device__ __forceinline__ f16x8 decode8_fp8(const uint2 v)
{
    if constexpr (E5) {
        const uint32_t w[2] = {v.x, v.y};
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            h[2 * i] = ((w[i] << 8) & 0xFF00u) | ((w[i] << 16) & 0xFF000000u);
            h[2 * i + 1] = ((w[i] >> 8) & 0xFF00u) | (w[i] & 0xFF000000u);
        }
        return __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
    } else {
        const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, false);
        const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, true);
        const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, false);
        const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, true);
        return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    }
}

// One operand's 16 byte codes (E4M3, or E5M2 when E5) -> FP16.
template <bool E5>
__device__ __forceinline__ void decode16_fp8(const uint4 v, f16x8& lo, f16x8& hi)
{
    if constexpr (E5)
        decode16_e5m2(v, lo, hi);
    else
        decode16(v, lo, hi);
}

// MXFP8: 16 E4M3 codes of one 32-element block -> two BF16 8-vectors of
// code * s, with s = 2^d (d <= 0) the block's scale relative to the
// reference exponent; exact whenever code * s is a BF16 number (every code
// for d >= -124; the GEMM's products need the stricter pair condition of
// its MX prologue).
__device__ __forceinline__ void decode16(const uint4 v, float s, bf16x8& lo, bf16x8& hi)
{
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, s, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, s, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, s, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, s, true);
    const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.z, s, false);
    const bf16x2 f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.z, s, true);
    const bf16x2 g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.w, s, false);
    const bf16x2 h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.w, s, true);
    lo = bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    hi = bf16x8{e[0], e[1], f[0], f[1], g[0], g[1], h[0], h[1]};
}

// MXFP8: 8 E4M3 codes -> BF16 8-vector of code * s (the lower or upper half
// of what decode16 with a scale returns for 16 codes).
__device__ __forceinline__ bf16x8 decode8_mx(const uint2 v, float s)
{
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, s, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, s, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, s, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, s, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E8M0 helper: the converter scale 2^(c - ref) (c <= ref) as an FP32 power
// of two.  The converters read only the exponent field of their scale
// operand (checked on gfx950: every pair of codes at every exponent field
// 0..254 gives the same result with mantissa bits 0, 1, 2^22 and 2^23 - 1),
// so below 2^-126 the denormal or zero that ldexp returns (field 0) acts as
// 2^-127, the clamp the decode needs.  Two instructions with the byte
// extract, against four for forming the field by hand.
__device__ __forceinline__ float e8m0_rel(uint32_t c, uint32_t ref)
{
    return __builtin_ldexpf(1.0f, (int)c - (int)ref);
}

// Two FP32 values -> packed BF16 pair (first in the low half) by the
// hardware converter v_cvt_pk_bf16_f32: round to nearest even, NaN to a quiet
// NaN; equal to RNE on the bits for all 2^32 inputs (checked exhaustively on
// gfx950).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b)
{
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// NVFP4: 32 E2M1 codes (one 16-byte LDS read of a lane) -> four FP16
// 8-vectors, word g holding the codes of MFMA k-step g; each code is
// multiplied by its 16-block's E4M3 scale (s01: the scales of words 0-1 and
// 2-3).  E2M1 * E4M3 lies in {0} u [2^-10, 2688] with at most 6 significant
// bits, so every product is an exact FP16 value.
__device__ __forceinline__ f16x8 decode_nv_word(uint32_t w, _Float16 s)
{
    const f16x2 ss = {s, s};
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Workgroup shapes: NWM x NWN waves, each owning (32*TI) x 64 outputs.
template <int NWM_, int NWN_, int TI_>
struct Shape {
    static constexpr int NWM = NWM_, NWN = NWN_, TI = TI_, TJ = 2;
    static constexpr int BM = 32 * TI * NWM, BN = 64 * NWN;
};
using ShapeDense = Shape<4, 2, 2>;      // 256 x 128, promoted modes
using ShapeWide = Shape<2, 4, 4>;       // 256 x 256, modes without promotion
using ShapeGrouped = Shape<2, 2, 2>;    // 128 x 128, MoE groups
using ShapeShort = Shape<2, 2, 1>;      // 64 x 128, MoE groups below kShortRows rows
constexpr int32_t kWideRows = 256;      // row groups this long take ShapeWide (exact path)
constexpr int32_t kShortRows = 64;      // row groups this short take ShapeShort

// SCW: scale words per tile row and K block staged with the codes (MX: the
// four E8M0 bytes; NVFP4: the eight E4M3 bytes as two words); word h of tile
// row rr (A rows, then B rows) at SCW_OFF + 4 (h (BM + BN) + rr).
template <class S, int ROW, bool B_TILE, bool A_TILE = false, int SCW = 0>
struct Lds {
    static constexpr int A_BYTES = S::BM * ROW;
    static constexpr int B_BYTES = S::BN * ROW;
    static constexpr int SB_BYTES = B_TILE ? S::BN * 4 : 0;                    // B 1x128 scales of the block
    static constexpr int SA_BYTES = A_TILE ? S::BM * 4 : 0;                    // A 1x128 scales
    static constexpr int SCW_OFF = A_BYTES + B_BYTES + SB_BYTES + SA_BYTES;
    static constexpr int STAGE = SCW_OFF + SCW * (S::BM + S::BN) * 4;
};

// Tile schedules: one dense problem; MoE groups of rows (each with its own
// B); MoE groups of the contraction (weight gradients, one C per group).
enum { GROUP_NONE = 0, GROUP_M = 1, GROUP_K = 2 };

// ELEMS (FP8 per-tensor operands only): bit 0 = A is E5M2, bit 1 = B is E5M2.
// MMA8: accumulate on the FP8 matrix instructions (v_mfma_scale_*_f8f6f4)
// instead of the exact FP16/BF16 decode: the codes go from LDS straight into
// the MFMA, MX scales are applied by the instruction, and the 1x128 / 128x128
// promotion stays as above.  The instruction's own sum is not exact (see the
// header), so its results are bounded more loosely than the default path's.
// Four-wave workgroups (the MoE tile) run two to a CU: declaring it caps them
// at 256 VGPRs, which puts their MFMA results in VGPRs rather than AGPRs, so
// the promotion reads the partial sums without a copy out of the AGPRs.
template <class S, int AMODE, int BMODE, bool OUT_BF16, int GROUP, int ELEMS = 0, bool MMA8 = false>
__global__ __launch_bounds__(64 * S::NWM * S::NWN, S::NWM * S::NWN == 4 ? 2 : 1) void gemm_block_scaled_kernel(GemmParams p)
{
    constexpr int NWM = S::NWM, NWN = S::NWN;
    constexpr int NW = NWM * NWN;        // waves
    constexpr int NT = 64 * NW;          // threads
    constexpr int BM = S::BM, BN = S::BN;
    constexpr int TI = S::TI;            // sub-tiles along m per wave
    constexpr int TJ = S::TJ;            // sub-tiles along n per wave
    constexpr int WM = 32 * TI;
    constexpr bool PROMOTE = !(AMODE == FGS_SCALE_TENSOR && BMODE == FGS_SCALE_TENSOR) &&
                             AMODE != FGS_SCALE_NV16_E4M3 && AMODE != FGS_SCALE_MX32_E8M0;
    constexpr bool B_TILE = BMODE == FGS_SCALE_TILE_1x128;
    constexpr bool MX = AMODE == FGS_SCALE_MX32_E8M0;
    // promoted modes at the 256 x 256 tile: 16x16 output tiles whose partial
    // sums over one scale block are formed and promoted one tile at a time,
    // so no partial-sum array has to live across the block (it would not fit
    // beside 128 accumulators at two waves per SIMD).  On the FP8
    // instructions one 16x16x128 MFMA is the block; on the exact path four
    // chained 16x16x32 FP16 MFMAs, the B fragments decoded once per block.
    constexpr bool MMA16 = PROMOTE && TI == 4;
    // the exact path's software-pipelined K loop: dense GEMMs in every mode
    // but the promoted 16x16 tiles and NVFP4.  The MoE schedules keep the
    // per-k-step loop, which skips the fragments of rows a group does not
    // own (measured: 389 against 280 TFLOP/s on the MoE layers)
    constexpr bool PIPE = ((AMODE == FGS_SCALE_TENSOR || AMODE == FGS_SCALE_MX32_E8M0) && !PROMOTE ||
                           PROMOTE && !MMA16) && !MMA8 && GROUP == GROUP_NONE;
    // MMA16 with 1x128 A scales stages them in LDS with the codes (eight
    // rows per lane would not fit in registers)
    constexpr bool A_LDS = MMA16 && AMODE == FGS_SCALE_TILE_1x128;
    constexpr bool NV = AMODE == FGS_SCALE_NV16_E4M3;
    // staged row: 128 K-elements = 128 bytes (E4M3) or 64 bytes (E2M1)
    constexpr int ROW = NV ? 64 : 128;
    constexpr int CPR = ROW / 16;            // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;            // rows per DMA wave-instruction (1 KiB)
    constexpr int SH = CPR == 8 ? 1 : 2;     // swizzle: slot = chunk ^ ((row >> SH) & (CPR - 1))
    constexpr int SCW = MX ? 1 : (NV ? 2 : 0);    // block-scale words per tile row staged in LDS
    using L = Lds<S, ROW, B_TILE, A_LDS, SCW>;
    static_assert(!(BMODE == FGS_SCALE_BLOCK_128x128 && BN % 128 != 0), "128x128 B blocks need 128-aligned tiles");
    static_assert(BN / 64 <= NW, "B 1x128 scale staging needs BN / 64 waves");
    static_assert(!A_LDS || BM / 64 <= NW, "A 1x128 scale staging needs BM / 64 waves");
    static_assert((BM + BN) % 64 == 0, "scale-word staging takes 64 tile rows per wave-instruction");

    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_scan[NT];
    __shared__ int s_sel[2];
    // MX: reference E8M0 byte of every A row and B row of the tile (largest
    // non-NaN scale byte over all of K), NaN-scale flags, the B tile's reference
    __shared__ uint8_t s_mx_ref[AMODE == FGS_SCALE_MX32_E8M0 ? BM + BN : 1];
    __shared__ uint8_t s_mx_nan[AMODE == FGS_SCALE_MX32_E8M0 ? BM + BN : 1];
    __shared__ uint32_t s_mx_eb;

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int wm = w / NWN, wn = w % NWN;   // wave grid NWM x NWN

    // ------------------------------------------------------------ tile --
    int64_t m0, m_end, n0;
    const uint8_t* Ap = p.A;
    const float* sAp = p.sA;
    const uint8_t* Bp = p.B;
    const float* sBp = p.sB;
    int64_t nkb = p.K / BK;
    // contraction groups: tokens of the group's last K block (1 .. BK); the
    // k-steps past them multiply zero codes and are skipped
    int kv_last = BK;
    int64_t c_off = 0;                    // elements from C to this tile's C matrix
    if constexpr (GROUP == GROUP_NONE) {
        int id = blockIdx.x;
        const int T = p.tiles_m * p.tiles_n;
        // workgroups are dealt round-robin to the 8 XCDs: give each XCD a
        // contiguous range of the tile order so its L2 sees neighbouring tiles
        if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
        // the order runs down GM m-tiles, then to the next n-tile: with 32
        // workgroups per XCD in flight, GM = 4 keeps about 4 A panels and 8
        // B panels live in the XCD's L2 (on the Llama-3-8B step, same box:
        // GM 4 1263-1287 TFLOP/s, 2 or 6 1255-1260, 8 1228-1276, 16 1184-1222)
        const int GM = 4;
        const int group = id / (GM * p.tiles_n);
        const int first_m = group * GM;
        const int gsz = min(p.tiles_m - first_m, GM);
        const int in_group = id % (GM * p.tiles_n);
        const int tm = first_m + in_group % gsz;
        const int tn = in_group / gsz;
        m0 = (int64_t)tm * BM;
        m_end = p.M;
        n0 = (int64_t)tn * BN;
    } else if constexpr (GROUP == GROUP_M) {
        // Device-side schedule over the tiles of all groups in canonical
        // order u (group, then n-tile, then m-tile fastest).  Workgroups are
        // taken in blocks of 64, from the front of the order for even blocks
        // and from the back for odd ones, so short (HBM-bound) and long
        // (MFMA-bound) groups run side by side whatever order the groups come
        // in.  Within a full block, workgroup 8 r + x (dealt to XCD x) takes
        // the block's tile 8 x + r: an XCD gets 8 consecutive tiles, the
        // m-tiles of one n-tile, which read the same weight rows through its
        // L2 (8 XCDs each fetching them measured 5x the weight bytes on the
        // DeepSeek-V3 long groups).  The last, partial block keeps the plain
        // order.  v -> u is a bijection on [0, T): the front takes [0, F) and
        // the back [T - B, T) with F + B = T.
        auto m_tiles = [&](int g) {
            int cnt = 0;
            if (g < p.G) {
                const int32_t o0 = p.offsets[g], o1 = p.offsets[g + 1];
                if (o0 >= 0 && o1 >= o0 && o1 <= p.M && o1 - o0 >= p.grp_lo && o1 - o0 < p.grp_hi)
                    cnt = (o1 - o0 + BM - 1) / BM;
            }
            return cnt;
        };
        // Prefix sums of the groups' tile counts, NT groups at a time: an
        // inclusive scan inside each wave (shuffles, no barrier), then the
        // wave totals through LDS (two barriers per chunk of groups).
        // Returns the chunk's total; cnt and excl are this thread's group's
        // count and exclusive prefix within the chunk.
        auto chunk_scan = [&](int chunk, int& cnt, int& excl) -> int {
            cnt = m_tiles(chunk + t);
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(incl, d);
                if (l >= d) incl += y;
            }
            if (l == 63) s_scan[w] = incl;
            __syncthreads();
            int before = 0, all = 0;
            for (int i = 0; i < NW; ++i) {
                const int c = s_scan[i];
                all += c;
                if (i < w) before += c;
            }
            __syncthreads();                          // s_scan is written again by the next chunk
            excl = before + incl - cnt;
            return all;
        };
        if (t == 0) s_sel[0] = -1;                    // ordered before any pick by the scan's barriers
        int total_tiles = 0, cnt0 = 0, excl0 = 0, all0 = 0;
        for (int chunk = 0; chunk < p.G; chunk += NT) {
            int cnt, excl;
            const int all = chunk_scan(chunk, cnt, excl);
            if (chunk == 0) {
                cnt0 = cnt;
                excl0 = excl;
                all0 = all;
            }
            total_tiles += all;
        }
        const int64_t total = (int64_t)total_tiles * p.tiles_n;
        if ((int64_t)blockIdx.x >= total) return;                  // beyond the last tile
        const int64_t bx = blockIdx.x, blk = bx >> 6;
        const int64_t inner = (blk + 1) * 64 <= total ? 8 * (bx & 7) + ((bx >> 3) & 7) : (bx & 63);
        const int64_t vbase = ((blk >> 1) << 6) + inner;
        const int64_t v = (blk & 1) ? total - 1 - vbase : vbase;
        // the group that holds tile v (exactly one thread finds it); the
        // first chunk's scan is reused, later chunks are scanned again
        int running = 0;
        for (int chunk = 0; chunk < p.G; chunk += NT) {
            int cnt = cnt0, excl = excl0, all = all0;
            if (chunk > 0) all = chunk_scan(chunk, cnt, excl);
            const int ex = running + excl;
            if (cnt > 0 && v >= (int64_t)ex * p.tiles_n && v < (int64_t)(ex + cnt) * p.tiles_n) {
                s_sel[0] = chunk + t;
                s_sel[1] = ex;
            }
            running += all;
        }
        __syncthreads();
        const int g = s_sel[0];
        if (g < 0) return;                                    // unreachable for v < total
        const int32_t o0 = p.offsets[g], o1 = p.offsets[g + 1];
        const int mt_g = (o1 - o0 + BM - 1) / BM;
        const int64_t local = v - (int64_t)s_sel[1] * p.tiles_n;
        const int tn = (int)(local / mt_g), tm = (int)(local % mt_g);
        m0 = (int64_t)o0 + (int64_t)tm * BM;
        m_end = o1;
        n0 = (int64_t)tn * BN;
        Bp = p.B + (int64_t)g * p.b_group_stride;
        sBp = p.sB + (int64_t)g * p.sb_group_stride;
    } else {
        // Contraction groups: group g owns the 128-token blocks
        // floor(o_g / 128) + g .. + ceil(M_g / 128) - 1 of both operands (the
        // layout of the per-group column-wise quantizer) and the C matrix at
        // g * M * ldc.  Workgroups run group by group; within a group of
        // per % 8 == 0 tiles, the eight XCDs (dealt workgroups round-robin)
        // each take a contiguous eighth of the tile order.  The order runs
        // down GM m-tiles, then to the next n-tile, and sets the shape of the
        // region of C that an XCD's tiles in flight write.  Measured on
        // DeepSeek-V3, same box: gate/up dW [4096 x 7168] (56 n-tiles) 7.45-
        // 7.47 ms with GM = 2, 7.62-7.67 with 1, 7.94-8.11 with 8; down dW
        // [7168 x 2048] (16 n-tiles) 3.56-3.61 ms with GM = 16, 3.57 with 8,
        // 3.76 with 4, 4.22 with 2, 4.53 with 1.  A group without tokens, or
        // with offsets out of order or range, runs no K block and writes
        // zeros.
        const int64_t per = (int64_t)p.tiles_m * p.tiles_n;
        const int g = (int)(blockIdx.x / per);
        int id = (int)(blockIdx.x % per);
        if ((per & 7) == 0) id = (id & 7) * (int)(per >> 3) + (id >> 3);
        const int GM = p.tiles_n >= 32 ? 2 : 8;
        const int group = id / (GM * p.tiles_n);
        const int first_m = group * GM;
        const int gsz = min(p.tiles_m - first_m, GM);
        const int in_group = id % (GM * p.tiles_n);
        m0 = (int64_t)(first_m + in_group % gsz) * BM;
        m_end = p.M;
        n0 = (int64_t)(in_group / gsz) * BN;
        const int32_t o0 = p.offsets[g], o1 = p.offsets[g + 1];
        const bool ok = o0 >= 0 && o1 >= o0 && (int64_t)o1 <= p.T;
        const int64_t kb0 = ok ? (int64_t)(o0 >> 7) + g : 0;
        nkb = ok ? (o1 - o0 + BK - 1) / BK : 0;
        if (nkb > 0) kv_last = (int)((o1 - o0) - (nkb - 1) * BK);
        Ap = p.A + kb0 * BK;
        Bp = p.B + kb0 * BK;
        sAp = p.sA + kb0 * p.M;
        sBp = p.sB + kb0 * p.N;
        c_off = (int64_t)g * p.M * p.ldc;
    }

    // ------------------------------------------------------- loaders --
    // wave w stages rows [A_ROWS*w, A_ROWS*(w+1)) of A and [B_ROWS*w, ...)
    // of B, RPI rows per wave-instruction; lane l fills slot l % CPR of row
    // rbase + l / CPR with chunk (l % CPR) ^ ((row >> SH) & (CPR - 1)).  Rows
    // past the end are clamped (their products land in rows/columns never
    // stored).
    constexpr int A_ROWS = BM / NW, B_ROWS = BN / NW;
    constexpr int A_INSTR = A_ROWS / RPI, B_INSTR = B_ROWS / RPI;
    static_assert(A_INSTR >= 1 && B_INSTR >= 1, "tile too small for the wave count");
    const int srow = l / CPR, sslot = l % CPR;
    // per-lane byte offsets from the tile's first A / B row (row clamped,
    // < 256 rows x a row stride below 2^24 bytes, so 32 bits), and the
    // tile's uniform bases; a K block adds kb * ROW to the bases
    uint32_t a_off[A_INSTR], b_off[B_INSTR];
#pragma unroll
    for (int u = 0; u < A_INSTR; ++u) {
        const int lr = A_ROWS * w + RPI * u + srow;
        int64_t r = m0 + lr;
        r = r < m_end ? r : m_end - 1;
        a_off[u] = (uint32_t)((r - m0) * p.lda) + 16 * (sslot ^ ((lr >> SH) & (CPR - 1)));
    }
#pragma unroll
    for (int u = 0; u < B_INSTR; ++u) {
        const int lr = B_ROWS * w + RPI * u + srow;
        int64_t r = n0 + lr;
        r = r < p.N ? r : p.N - 1;
        b_off[u] = (uint32_t)((r - n0) * p.ldb) + 16 * (sslot ^ ((lr >> SH) & (CPR - 1)));
    }
    const uint8_t* a_base = uniform_ptr(Ap + m0 * p.lda);
    const uint8_t* b_base = uniform_ptr(Bp + n0 * p.ldb);
    // LDS addresses (M0) of the stages and of this wave's A and B rows
    const uint32_t lds0 = lds_offset(smem);
    const uint32_t lds_a = __builtin_amdgcn_readfirstlane((uint32_t)(A_ROWS * w * ROW));
    const uint32_t lds_b = __builtin_amdgcn_readfirstlane((uint32_t)(L::A_BYTES + B_ROWS * w * ROW));
    int64_t sb_col = n0 + 64 * (w % (BN / 64)) + l;   // B 1x128 scales: waves 0 .. BN/64-1 stage 64 each
    sb_col = sb_col < p.N ? sb_col : p.N - 1;
    // A 1x128 scales (A_LDS): waves NW - BM/64 .. NW-1 stage 64 rows each
    constexpr int SAW0 = NW - BM / 64;
    int64_t sa_row = m0 + 64 * ((w - SAW0) & (BM / 64 - 1)) + l;
    sa_row = sa_row < m_end ? sa_row : m_end - 1;
    // MX / NVFP4 block scales: wave-instruction u (of SC_INSTR per stage,
    // wave w issuing u = w, w + NW, ..) stages word u / (tile rows / 64) of
    // the 128-K block's scale bytes of tile rows 64 (u % (rows / 64)) + l,
    // A rows first, then B rows (clamped), so the fragment loop reads its
    // scales from LDS instead of one scattered 4-byte global load per lane.
    constexpr int SC_ROWS = BM + BN, SC_INSTR = SCW * SC_ROWS / 64;
    constexpr int SC_PER_W = SCW ? (SC_INSTR + NW - 1) / NW : 1;
    const int64_t sc_row_bytes = MX ? p.K / 32 : p.K / 16;     // scale bytes of a row
    const uint8_t* sc_src[SC_PER_W];
    int sc_dst[SC_PER_W];
#pragma unroll
    for (int k = 0; k < SC_PER_W; ++k) {
        const int u = w + NW * k, blk = u % (SC_ROWS / 64), h = u / (SC_ROWS / 64);
        const int rr = 64 * blk + l;
        const uint8_t* base;
        if (rr < BM) {
            const int64_t r = m0 + rr < m_end ? m0 + rr : m_end - 1;
            base = reinterpret_cast<const uint8_t*>(p.sA) + r * sc_row_bytes;
        } else {
            const int64_t r = n0 + rr - BM < p.N ? n0 + rr - BM : p.N - 1;
            base = reinterpret_cast<const uint8_t*>(sBp) + r * sc_row_bytes;
        }
        sc_src[k] = base + 4 * h;
        sc_dst[k] = L::SCW_OFF + 4 * (h * SC_ROWS + 64 * blk);
    }

    // Rows of the tile that exist; a wave-instruction whose rows all lie past
    // them is not issued (its LDS rows only feed outputs that are never
    // stored), and waves whose accumulator rows all lie past them skip the
    // MFMAs: short MoE groups then move and multiply only what they own.
    const int a_live = (int)(m_end - m0 < BM ? m_end - m0 : BM);
    const int b_live = (int)(p.N - n0 < BN ? p.N - n0 : BN);
    const bool wave_live = WM * wm < a_live;
    auto stage_block = [&](int64_t kb, int stage) {
        uint8_t* st = smem + stage * L::STAGE;
        const int64_t ko = kb * ROW;
        const uint32_t lst = lds0 + (uint32_t)(stage * L::STAGE);
#pragma unroll
        for (int u = 0; u < A_INSTR; ++u)
            if (A_ROWS * w + RPI * u < a_live) g2lds16_s(a_base + ko, a_off[u], lst + lds_a + RPI * u * ROW);
#pragma unroll
        for (int u = 0; u < B_INSTR; ++u)
            if (B_ROWS * w + RPI * u < b_live) g2lds16_s(b_base + ko, b_off[u], lst + lds_b + RPI * u * ROW);
        if constexpr (B_TILE)
            if (w < BN / 64) g2lds4(sBp + kb * p.N + sb_col, st + L::A_BYTES + L::B_BYTES + 256 * w);
        if constexpr (A_LDS)
            if (w >= SAW0) g2lds4(sAp + kb * p.M + sa_row, st + L::A_BYTES + L::B_BYTES + L::SB_BYTES + 256 * (w - SAW0));
        if constexpr (SCW > 0) {
#pragma unroll
            for (int k = 0; k < SC_PER_W; ++k)
                if (w + NW * k < SC_INSTR) g2lds4(sc_src[k] + 4 * SCW * kb, st + sc_dst[k]);
        }
    };

    // rows of this lane's accumulators: m = m0 + WM*wm + 32*i + (l & 31)
    int64_t am[TI];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int64_t m = m0 + WM * wm + 32 * i + (l & 31);
        am[i] = m < m_end ? m : m_end - 1;
    }

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // MXFP8 scales.  A (per lane row m): E_A[m] = the largest E8M0 byte of
    // the row over all of K; B: one E_B for the tile (the largest byte of its
    // rows over all of K).  Every code is decoded as code * 2^(e - E) into
    // BF16 and the FP16/BF16 matrix unit sums the products over all of K in
    // FP32; the epilogue multiplies by 2^(E_A + E_B - 254) (exact scaling),
    // so no per-block promotion is needed.  Exact whenever every pair of
    // blocks that meet has (e_A - E_A) + (e_B - E_B) >= -108: both decoded
    // codes are then BF16 numbers and their product, at least
    // 2^-9 2^-9 2^-108 = 2^-126, a normal FP32 number.  A pair further apart
    // holds products below 448^2 2^-108 < 2^-90 reference units, and what it
    // adds (rounded, flushed, or with the converter's scale saturated at
    // 2^-127 for blocks more than 127 below the reference) stays below that.  NaN scale bytes (0xFF) are left out of the references and
    // flagged: their rows (A) and columns (B) of C are NaN, as in the
    // dequantized product.  The four bytes of a row's 128-K block are one
    // aligned 32-bit word.
    int64_t bn[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int64_t n = n0 + 64 * wn + 32 * j + (l & 31);
        bn[j] = n < p.N ? n : p.N - 1;
    }
    uint32_t ea[TI], eb = 0;
    if constexpr (MX && !MMA8) {
        // the tile's rows: A rows 0 .. BM-1, then B rows (rows past the end
        // clamped; they only feed outputs that are never stored): their
        // references formed once per launch by mx_row_ref_kernel when the
        // caller brought a workspace, else scanned here, one row per thread
        if (t == 0) s_mx_eb = 0;
        __syncthreads();
        const uint8_t* const sA8 = reinterpret_cast<const uint8_t*>(p.sA);
        const uint8_t* const sB8 = reinterpret_cast<const uint8_t*>(sBp);
        const int64_t ksc = p.K / 32;                 // scale bytes of a row
        // 16 bytes per load where the rows allow it, eight loads in flight
        // before any is scanned (the eight 405B MXFP8 GEMMs, same box: 7%
        // less time than 4-byte loads each waited for before the next; the
        // per-launch pass saves 10%)
        const bool wide_rows = (ksc & 15) == 0 && (reinterpret_cast<uintptr_t>(sA8) & 15) == 0 &&
                               (reinterpret_cast<uintptr_t>(sB8) & 15) == 0;
        for (int rr = t; rr < BM + BN; rr += NT) {
            const bool is_a = rr < BM;
            int64_t row = is_a ? m0 + rr : n0 + (rr - BM);
            const int64_t lim = is_a ? m_end : p.N;
            row = row < lim ? row : lim - 1;
            uint32_t mref = 0, nan = 0;
            if (p.mx_ref) {
                const uint32_t v = p.mx_ref[is_a ? row : p.M + row];
                mref = v & 0xFFu;
                nan = v >> 8;
            } else {
                auto scan_word = [&](uint32_t w4) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t v = (w4 >> (8 * b)) & 0xFFu;
                        nan |= v == 0xFFu;
                        mref = max(mref, v == 0xFFu ? 0u : v);
                    }
                };
                const uint8_t* const rowp = (is_a ? sA8 : sB8) + row * ksc;
                if (wide_rows) {
                    constexpr int BATCH = 8;
                    const uint4* src = reinterpret_cast<const uint4*>(rowp);
                    const int64_t n16 = ksc / 16;
                    int64_t c = 0;
                    for (; c + BATCH <= n16; c += BATCH) {
                        uint4 q[BATCH];
#pragma unroll
                        for (int k = 0; k < BATCH; ++k) q[k] = src[c + k];
#pragma unroll
                        for (int k = 0; k < BATCH; ++k) {
                            scan_word(q[k].x);
                            scan_word(q[k].y);
                            scan_word(q[k].z);
                            scan_word(q[k].w);
                        }
                    }
                    for (; c < n16; ++c) {
                        const uint4 q = src[c];
                        scan_word(q.x);
                        scan_word(q.y);
                        scan_word(q.z);
                        scan_word(q.w);
                    }
                } else {
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(rowp);
                    for (int64_t c = 0; c < ksc / 4; ++c) scan_word(src[c]);
                }
            }
            s_mx_ref[rr] = (uint8_t)mref;
            s_mx_nan[rr] = (uint8_t)nan;
            if (!is_a) atomicMax(&s_mx_eb, mref);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TI; ++i) ea[i] = s_mx_ref[WM * wm + 32 * i + (l & 31)];
        eb = s_mx_eb;
    }
    // NVFP4 scales: the eight E4M3 bytes of a fragment row's 128-K block are
    // two aligned 32-bit words (16-blocks 0-3 and 4-7), staged in LDS

    // prologue: block 0 -> stage 0
    if (nkb > 0) stage_block(0, 0);
    float sa_next[TI];
    if constexpr (AMODE == FGS_SCALE_TILE_1x128 && !A_LDS) {
#pragma unroll
        for (int i = 0; i < TI; ++i) sa_next[i] = nkb > 0 ? sAp[am[i]] : 0.0f;
    }
    float sb_next = 0.0f;
    // 128x128 B blocks: a wave's 64 columns lie in one block (clamped for
    // waves past N, whose columns are never stored)
    int64_t sb_row = (n0 + 64 * wn) / 128;
    if (sb_row > (p.N - 1) / 128) sb_row = (p.N - 1) / 128;
    if constexpr (BMODE == FGS_SCALE_BLOCK_128x128) if (nkb > 0) sb_next = sBp[sb_row * nkb];
    wait_lds_dma();
    __syncthreads();

    // fragment read offsets: row R = base + (l & 31) (base a multiple of
    // 32) has (R >> SH) & (CPR - 1) == (l >> SH) & (CPR - 1); chunk c of the
    // row lives in slot c ^ swz
    const int swz = (l >> SH) & (CPR - 1), half = l >> 5;

    if constexpr (PIPE) {
        // One scale per operand (or MX, whose block scales are applied in the
        // decode relative to per-row and per-tile reference exponents): no
        // promotion, so a block is eight 32x32x16 k-steps (ks, h) straight
        // into the accumulators.  Lane half `half`
        // reads chunk 2 ks + half of its rows; bytes 0-7 feed k-step (ks, 0),
        // bytes 8-15 k-step (ks, 1).  The decode runs half a k-step ahead of
        // the matrix instructions, one operand fragment per MFMA: under the
        // MFMAs of (ks, 0) the codes of (ks, 1) are decoded, under (ks, 1)
        // those of (ks + 1, 0).  A fragment's next 16-byte chunk is read from
        // LDS as soon as the current one is decoded: one 16-byte read per
        // lane, for which the swizzled layout is free of bank conflicts (two
        // 8-byte reads per chunk are not).  The block's last k-step
        // runs after the barrier that publishes the next stage, so the next
        // block's first decode hides under it too; by then no wave reads the
        // current stage any more, which the next block's loads overwrite.
        constexpr bool E5A = (ELEMS & 1) != 0, E5B = (ELEMS & 2) != 0;
        constexpr int NP = TI + TJ, NT = TI * TJ, LAG = NT > NP ? NT - NP : 1;
        static_assert(NP <= NT, "one fragment decode per MFMA");
        using Frag = std::conditional_t<MX, bf16x8, f16x8>;
        Frag af[TI][2], bf[TJ][2];
        uint4 raw[NP];
        uint32_t sw[MX ? NP : 1] = {};   // MX: the fragments' rows' scale words of the block
        auto rdsw = [&](int stage) {
            if constexpr (MX) {
                const uint32_t* scw = reinterpret_cast<const uint32_t*>(smem + stage * L::STAGE + L::SCW_OFF);
#pragma unroll
                for (int pc = 0; pc < NP; ++pc)
                    sw[pc] = scw[pc < TI ? WM * wm + 32 * pc + (l & 31) : BM + 64 * wn + 32 * (pc - TI) + (l & 31)];
            }
        };
        auto rd = [&](int stage, int pc, int ks) -> uint4 {
            const uint8_t* st = smem + stage * L::STAGE;
            const uint8_t* q = pc < TI ? st + (WM * wm + (l & 31) + 32 * pc) * ROW
                                       : st + L::A_BYTES + (64 * wn + (l & 31) + 32 * (pc - TI)) * ROW;
            return *reinterpret_cast<const uint4*>(q + (((2 * ks + half) ^ swz) << 4));
        };
        // k-step (ks, h) of fragment pc from the chunk in raw[pc]
        auto dec = [&](int pc, int h, int ks) {
            const uint2 v = h == 0 ? make_uint2(raw[pc].x, raw[pc].y) : make_uint2(raw[pc].z, raw[pc].w);
            if constexpr (MX) {
                // k-steps (ks, 0) and (ks, 1) both lie in MX block ks of the row
                const float sc = e8m0_rel((sw[pc] >> (8 * ks)) & 0xFFu, pc < TI ? ea[pc] : eb);
                if (pc < TI) af[pc][h] = decode8_mx(v, sc);
                else bf[pc - TI][h] = decode8_mx(v, sc);
            } else {
                if (pc < TI) af[pc][h] = decode8_fp8<E5A>(v);
                else bf[pc - TI][h] = decode8_fp8<E5B>(v);
            }
        };
        // promoted modes: each block's k-steps sum into part (the block's
        // first k-step starts from zero), promoted into acc after the last
        f32x16 part[PROMOTE ? TI : 1][PROMOTE ? TJ : 1];
        auto mma = [&](int t, int h, bool first) {
            const int i = t / TJ, j = t % TJ;
            if constexpr (PROMOTE)
                part[i][j] = mfma16(bf[j][h], af[i][h], first ? f32x16{} : part[i][j]);
            else
                acc[i][j] = mfma16(bf[j][h], af[i][h], acc[i][j]);
        };
        const float sa_t = AMODE == FGS_SCALE_TENSOR ? p.sA[0] : 1.0f;
        const float sb_t = BMODE == FGS_SCALE_TENSOR ? sBp[0] : 1.0f;
        float sa_cur[TI], sb_cur = 0.0f;
        float4 sbq[B_TILE ? 4 * TJ : 1];   // 1x128 B: the block's scales of this lane's columns
        auto promote = [&]() {
            if constexpr (PROMOTE) {
    #pragma unroll
                for (int i = 0; i < TI; ++i) {
                    const float fa = AMODE == FGS_SCALE_TENSOR ? sa_t : sa_cur[i];
    #pragma unroll
                    for (int j = 0; j < TJ; ++j)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            float f;
                            if constexpr (B_TILE) {
                                // column n = 64 wn + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4
                                const float4 q4 = sbq[4 * j + (r >> 2)];
                                const float sbv[4] = {q4.x, q4.y, q4.z, q4.w};
                                f = fa * sbv[r & 3];
                            } else {
                                f = fa * (BMODE == FGS_SCALE_TENSOR ? sb_t : sb_cur);
                            }
                            acc[i][j][r] = __builtin_fmaf(part[i][j][r], f, acc[i][j][r]);
                        }
                }
            }
        };
        if (wave_live && nkb > 0) {
            rdsw(0);
#pragma unroll
            for (int pc = 0; pc < NP; ++pc) raw[pc] = rd(0, pc, 0);
#pragma unroll
            for (int pc = 0; pc < NP; ++pc) dec(pc, 0, 0);
        }
        for (int64_t kb = 0; kb < nkb; ++kb) {
            const int cur = (int)(kb & 1);
            const bool more = kb + 1 < nkb;
            if constexpr (PROMOTE) {
    #pragma unroll
                for (int i = 0; i < TI; ++i) sa_cur[i] = AMODE == FGS_SCALE_TILE_1x128 ? sa_next[i] : 1.0f;
                sb_cur = sb_next;
            }
            if (more) {
                stage_block(kb + 1, cur ^ 1);
                if constexpr (PROMOTE && AMODE == FGS_SCALE_TILE_1x128) {
    #pragma unroll
                    for (int i = 0; i < TI; ++i) sa_next[i] = sAp[(kb + 1) * p.M + am[i]];
                }
                if constexpr (PROMOTE && BMODE == FGS_SCALE_BLOCK_128x128) sb_next = sBp[sb_row * nkb + kb + 1];
            }
            if (wave_live) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        if (ks == 3 && h == 1) continue;
                        // (ks, 0): decode (ks, 1), read chunk ks + 1;
                        // (ks, 1): decode (ks + 1, 0)
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            mma(t, h, ks == 0 && h == 0);
                            if (t < NP) {
                                dec(t, h ^ 1, h == 0 ? ks : ks + 1);
                                if (h == 0 && ks + 1 < 4) raw[t] = rd(cur, t, ks + 1);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                if constexpr (B_TILE) {
                    // read before the barrier: the next block's loads may
                    // overwrite this stage once every wave has passed it
                    const float* ssb = reinterpret_cast<const float*>(smem + cur * L::STAGE + L::A_BYTES + L::B_BYTES);
    #pragma unroll
                    for (int j = 0; j < TJ; ++j)
    #pragma unroll
                        for (int q = 0; q < 4; ++q)
                            sbq[4 * j + q] = *reinterpret_cast<const float4*>(ssb + 64 * wn + 32 * j + 8 * q + 4 * (l >> 5));
                }
            }
            wait_lds_dma();
            __syncthreads();
            if (wave_live && more) {
                rdsw(cur ^ 1);
#pragma unroll
                for (int pc = 0; pc < NP; ++pc) raw[pc] = rd(cur ^ 1, pc, 0);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    mma(t, 1, false);
                    const int pc = t - LAG;
                    if (pc >= 0 && pc < NP) dec(pc, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int pc = NT - LAG; pc < NP; ++pc) dec(pc, 0, 0);
            } else if (wave_live) {
#pragma unroll
                for (int t = 0; t < NT; ++t) mma(t, 1, false);
            }
            if (wave_live) promote();
        }
    } else
    for (int64_t kb = 0; kb < nkb; ++kb) {
        const int cur = (int)(kb & 1);
        const bool more = kb + 1 < nkb;
        // scales of this block (prefetched one block ahead)
        float sa[TI];
#pragma unroll
        for (int i = 0; i < TI; ++i) sa[i] = AMODE == FGS_SCALE_TILE_1x128 && !A_LDS ? sa_next[i] : 1.0f;
        const float sb_blk = sb_next;
        uint32_t a_sw[TI], b_sw[TJ], a_nw[TI][2], b_nw[TJ][2];
        if (more) {
            stage_block(kb + 1, cur ^ 1);
            if constexpr (AMODE == FGS_SCALE_TILE_1x128 && !A_LDS) {
#pragma unroll
                for (int i = 0; i < TI; ++i) sa_next[i] = sAp[(kb + 1) * p.M + am[i]];
            }
            if constexpr (BMODE == FGS_SCALE_BLOCK_128x128) sb_next = sBp[sb_row * nkb + kb + 1];
        }

        if (wave_live) {
            const uint8_t* st = smem + cur * L::STAGE;
            const uint8_t* la = st + (WM * wm + (l & 31)) * ROW;
            const uint8_t* lb = st + L::A_BYTES + (64 * wn + (l & 31)) * ROW;
            if constexpr (SCW > 0) {
                // this block's scale words of the lane's A and B rows (staged)
                const uint32_t* scw = reinterpret_cast<const uint32_t*>(st + L::SCW_OFF);
    #pragma unroll
                for (int h = 0; h < SCW; ++h) {
    #pragma unroll
                    for (int i = 0; i < TI; ++i) {
                        const uint32_t v = scw[h * SC_ROWS + WM * wm + 32 * i + (l & 31)];
                        if constexpr (MX) a_sw[i] = v; else a_nw[i][h] = v;
                    }
    #pragma unroll
                    for (int j = 0; j < TJ; ++j) {
                        const uint32_t v = scw[h * SC_ROWS + BM + 64 * wn + 32 * j + (l & 31)];
                        if constexpr (MX) b_sw[j] = v; else b_nw[j][h] = v;
                    }
                }
            }

            f32x16 part[TI][TJ];
            if constexpr (PROMOTE && !MMA16) {
    #pragma unroll
                for (int i = 0; i < TI; ++i)
    #pragma unroll
                    for (int j = 0; j < TJ; ++j)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
            }
            // lane half h reads chunk 2*ks + h (bytes 32*ks + 16*h .. +15) of its
            // row: the pair of k-steps (2ks, 2ks+1) then covers k = 32*ks ..
            // 32*ks+31 once, with the same k order for A and B
            if constexpr (NV) {
                // lane half h reads chunk 2*ks2 + h (32 codes, k = 64*ks2 + 32*h ..
                // +31); word g of it feeds MFMA k-step (ks2, g), whose 16-block is
                // 4*ks2 + 2*h + g/2
    #pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
                    const int co = ((2 * ks2 + half) ^ swz) << 4;
                    f16x2 sa2[TI], sb2[TJ];
                    uint4 ra[TI], rb[TJ];
    #pragma unroll
                    for (int i = 0; i < TI; ++i) {
                        sa2[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a_nw[i][ks2] >> (16 * half), 1.0f, false);
                        ra[i] = *reinterpret_cast<const uint4*>(la + 32 * i * ROW + co);
                    }
    #pragma unroll
                    for (int j = 0; j < TJ; ++j) {
                        sb2[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b_nw[j][ks2] >> (16 * half), 1.0f, false);
                        rb[j] = *reinterpret_cast<const uint4*>(lb + 32 * j * ROW + co);
                    }
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        f16x8 af[TI], bf[TJ];
    #pragma unroll
                        for (int i = 0; i < TI; ++i) {
                            const uint32_t wd = g == 0 ? ra[i].x : g == 1 ? ra[i].y : g == 2 ? ra[i].z : ra[i].w;
                            af[i] = decode_nv_word(wd, sa2[i][g >> 1]);
                        }
    #pragma unroll
                        for (int j = 0; j < TJ; ++j) {
                            const uint32_t wd = g == 0 ? rb[j].x : g == 1 ? rb[j].y : g == 2 ? rb[j].z : rb[j].w;
                            bf[j] = decode_nv_word(wd, sb2[j][g >> 1]);
                        }
    #pragma unroll
                        for (int i = 0; i < TI; ++i)
    #pragma unroll
                            for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16(bf[j], af[i], acc[i][j]);
                    }
                }
            } else if constexpr (MMA16) {
                // 16x16 output tiles: A sub-tile a (rows 16 a ..) x B sub-tile
                // b (columns 16 b ..) lands in acc[a / 2][b / 2] floats
                // 4 (2 (a % 2) + b % 2) .. +3.  Lane group g = l / 16 holds
                // chunk g in bytes 0-15 and chunk 4 + g in bytes 16-31 of its
                // row, for A and B alike.
                constexpr int FB = (ELEMS & 2) ? 1 : 0, FA = (ELEMS & 1) ? 1 : 0;
                const int r16 = l & 15, g4 = l >> 4;
                const int sw16 = (r16 >> SH) & (CPR - 1);
                const int c0 = (g4 ^ sw16) << 4, c1 = ((4 + g4) ^ sw16) << 4;
                const uint8_t* la16 = st + (WM * wm + r16) * ROW;
                const uint8_t* lb16 = st + L::A_BYTES + (64 * wn + r16) * ROW;
                // FP8: the codes as they are; exact: decoded to FP16 once per
                // block, k-step s of lane group g = its codes 8 s .. 8 s + 7
                i32x8 bfr[MMA8 ? 2 * TJ : 1];
                f16x8 bfh[MMA8 ? 1 : 2 * TJ][4];
    #pragma unroll
                for (int b = 0; b < 2 * TJ; ++b) {
                    const uint4 x = *reinterpret_cast<const uint4*>(lb16 + 16 * b * ROW + c0);
                    const uint4 y = *reinterpret_cast<const uint4*>(lb16 + 16 * b * ROW + c1);
                    if constexpr (MMA8) {
                        bfr[b] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
                    } else {
                        decode16(x, bfh[b][0], bfh[b][1]);
                        decode16(y, bfh[b][2], bfh[b][3]);
                    }
                }
                const float sa_t = AMODE == FGS_SCALE_TENSOR ? p.sA[0] : 1.0f;
                const float fb = BMODE == FGS_SCALE_TENSOR ? sBp[0] : (BMODE == FGS_SCALE_BLOCK_128x128 ? sb_blk : 1.0f);
                // B 1x128 scales of this lane's columns 64 wn + 16 b + 4 g4 .. +3
                float4 sbt[B_TILE ? 2 * TJ : 1];
                if constexpr (B_TILE) {
                    const float* ssb = reinterpret_cast<const float*>(st + L::A_BYTES + L::B_BYTES);
    #pragma unroll
                    for (int b = 0; b < 2 * TJ; ++b)
                        sbt[b] = *reinterpret_cast<const float4*>(ssb + 64 * wn + 16 * b + 4 * g4);
                }
                if constexpr (MMA8) {
    #pragma unroll
                for (int a = 0; a < 2 * TI; ++a) {
                    const uint4 x = *reinterpret_cast<const uint4*>(la16 + 16 * a * ROW + c0);
                    const uint4 y = *reinterpret_cast<const uint4*>(la16 + 16 * a * ROW + c1);
                    const i32x8 afr = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
                    float fa = sa_t;
                    if constexpr (A_LDS)
                        fa = reinterpret_cast<const float*>(st + L::A_BYTES + L::B_BYTES + L::SB_BYTES)[WM * wm + 16 * a + r16];
    #pragma unroll
                    for (int b = 0; b < 2 * TJ; ++b) {
                        const f32x4 pb = mfma8_k128<FB, FA>(bfr[b], afr);
                        const int sub = 4 * (2 * (a & 1) + (b & 1));
                        f32x16& ac = acc[a >> 1][b >> 1];
                        if constexpr (B_TILE) {
                            const float sbv[4] = {sbt[b].x, sbt[b].y, sbt[b].z, sbt[b].w};
    #pragma unroll
                            for (int e = 0; e < 4; ++e) ac[sub + e] = __builtin_fmaf(pb[e], fa * sbv[e], ac[sub + e]);
                        } else {
                            const float f = fa * fb;
    #pragma unroll
                            for (int e = 0; e < 4; ++e) ac[sub + e] = __builtin_fmaf(pb[e], f, ac[sub + e]);
                        }
                    }
                }
                } else {
                // Exact: chain b of sub-tile a is four dependent 16x16x32
                // FP16 MFMAs, and the vector work of the sub-tile rides
                // between them, about two instructions per MFMA, in an order
                // fixed by scheduling fences: under chain 0 the four FP16
                // quarters of the A fragment are decoded, each just before
                // the MFMA that takes it; under chain b > 0 the four sums of
                // chain b - 1 are promoted (and under chain 1 also those of
                // the previous sub-tile's last chain), one per MFMA, so no
                // promotion waits on the chain it reads.
                auto promote = [&](int a, int b, int e, const f32x4& v, float fa) {
                    f32x16& ac = acc[a >> 1][b >> 1];
                    const int sub = 4 * (2 * (a & 1) + (b & 1));
                    float f;
                    if constexpr (B_TILE) {
                        const float sbv[4] = {sbt[b].x, sbt[b].y, sbt[b].z, sbt[b].w};
                        f = fa * sbv[e];
                    } else {
                        f = fa * fb;
                    }
                    ac[sub + e] = __builtin_fmaf(v[e], f, ac[sub + e]);
                };
                f32x4 pq[2 * TJ], plast = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                float fa_prev = 0.0f;
                // the next sub-tile's codes are read as soon as the last
                // chain has taken the first two FP16 quarters, into their
                // registers
                uint4 xn = *reinterpret_cast<const uint4*>(la16 + c0);
                uint4 yn = *reinterpret_cast<const uint4*>(la16 + c1);
    #pragma unroll
                for (int a = 0; a < 2 * TI; ++a) {
                    const uint4 x = xn, y = yn;
                    float fa = sa_t;
                    if constexpr (A_LDS)
                        fa = reinterpret_cast<const float*>(st + L::A_BYTES + L::B_BYTES + L::SB_BYTES)[WM * wm + 16 * a + r16];
                    f16x8 afh[4];
    #pragma unroll
                    for (int b = 0; b < 2 * TJ; ++b) {
    #pragma unroll
                        for (int k4 = 0; k4 < 4; ++k4) {
                            if (b == 0) {
                                const uint4 v = k4 < 2 ? x : y;
                                afh[k4] = decode8_fp8<false>((k4 & 1) ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y));
                            }
                            pq[b] = mfma16x16(bfh[b][k4], afh[k4], k4 == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : pq[b]);
                            __builtin_amdgcn_sched_barrier(0);
                            if (b >= 1) promote(a, b - 1, k4, pq[b - 1], fa);
                            if (b == 1 && a >= 1) promote(a - 1, 2 * TJ - 1, k4, plast, fa_prev);
                            if (b == 2 * TJ - 1 && k4 == 1 && a + 1 < 2 * TI) {
                                xn = *reinterpret_cast<const uint4*>(la16 + 16 * (a + 1) * ROW + c0);
                                yn = *reinterpret_cast<const uint4*>(la16 + 16 * (a + 1) * ROW + c1);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    plast = pq[2 * TJ - 1];
                    fa_prev = fa;
                }
    #pragma unroll
                for (int e = 0; e < 4; ++e) promote(2 * TI - 1, 2 * TJ - 1, e, plast, fa_prev);
                }
            } else if constexpr (MMA8) {
                // two 64-deep k-steps; lane half h holds chunk 4*s2 + h of its
                // row in bytes 0-15 and chunk 4*s2 + 2 + h in bytes 16-31, so
                // the instruction's first scale block is MX block 2*s2 (chunks
                // 4*s2, 4*s2 + 1) and its second MX block 2*s2 + 1; lane half
                // h supplies the scale of block 2*s2 + h.  Same for A and B.
                constexpr int FB = (ELEMS & 2) ? 1 : 0, FA = (ELEMS & 1) ? 1 : 0;
    #pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    if (GROUP == GROUP_K && kb == nkb - 1 && 64 * s2 >= kv_last) continue;
                    const int c0 = ((4 * s2 + half) ^ swz) << 4, c1 = ((4 * s2 + 2 + half) ^ swz) << 4;
                    i32x8 af[TI], bf[TJ];
                    int ea8[TI], eb8[TJ];
    #pragma unroll
                    for (int j = 0; j < TJ; ++j) {
                        const uint4 x = *reinterpret_cast<const uint4*>(lb + 32 * j * ROW + c0);
                        const uint4 y = *reinterpret_cast<const uint4*>(lb + 32 * j * ROW + c1);
                        bf[j] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
                        eb8[j] = MX ? (int)((b_sw[j] >> (8 * (2 * s2 + half))) & 0xFFu) : 127;
                    }
    #pragma unroll
                    for (int i = 0; i < TI; ++i) {
                        const uint4 x = *reinterpret_cast<const uint4*>(la + 32 * i * ROW + c0);
                        const uint4 y = *reinterpret_cast<const uint4*>(la + 32 * i * ROW + c1);
                        af[i] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
                        ea8[i] = MX ? (int)((a_sw[i] >> (8 * (2 * s2 + half))) & 0xFFu) : 127;
                    }
    #pragma unroll
                    for (int i = 0; i < TI; ++i)
    #pragma unroll
                        for (int j = 0; j < TJ; ++j) {
                            if constexpr (PROMOTE)
                                part[i][j] = mfma8<FB, FA>(bf[j], af[i], part[i][j], eb8[j], ea8[i]);
                            else
                                acc[i][j] = mfma8<FB, FA>(bf[j], af[i], acc[i][j], eb8[j], ea8[i]);
                        }
                }
            } else
    #pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (GROUP == GROUP_K && kb == nkb - 1 && 32 * ks >= kv_last) continue;
                const int co = ((2 * ks + half) ^ swz) << 4;
                if constexpr (MX) {
                    // k-steps 2ks, 2ks+1 are MX block ks of this 128-K block
                    bf16x8 af[TI][2], bf[TJ][2];
    #pragma unroll
                    for (int j = 0; j < TJ; ++j)
                        decode16(*reinterpret_cast<const uint4*>(lb + 32 * j * ROW + co),
                                 e8m0_rel((b_sw[j] >> (8 * ks)) & 0xFFu, eb), bf[j][0], bf[j][1]);
    #pragma unroll
                    for (int i = 0; i < TI; ++i)
                        decode16(*reinterpret_cast<const uint4*>(la + 32 * i * ROW + co),
                                 e8m0_rel((a_sw[i] >> (8 * ks)) & 0xFFu, ea[i]), af[i][0], af[i][1]);
    #pragma unroll
                    for (int h = 0; h < 2; ++h)
    #pragma unroll
                        for (int i = 0; i < TI; ++i)
    #pragma unroll
                            for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16(bf[j][h], af[i][h], acc[i][j]);
                } else {
                    f16x8 af[TI][2], bf[TJ][2];
    #pragma unroll
                    for (int j = 0; j < TJ; ++j)
                        decode16_fp8<(ELEMS & 2) != 0>(*reinterpret_cast<const uint4*>(lb + 32 * j * ROW + co), bf[j][0], bf[j][1]);
    #pragma unroll
                    for (int i = 0; i < TI; ++i)
                        decode16_fp8<(ELEMS & 1) != 0>(*reinterpret_cast<const uint4*>(la + 32 * i * ROW + co), af[i][0], af[i][1]);
    #pragma unroll
                    for (int h = 0; h < 2; ++h)
    #pragma unroll
                        for (int i = 0; i < TI; ++i)
    #pragma unroll
                            for (int j = 0; j < TJ; ++j) {
                                if constexpr (PROMOTE)
                                    part[i][j] = mfma16(bf[j][h], af[i][h], part[i][j]);
                                else
                                    acc[i][j] = mfma16(bf[j][h], af[i][h], acc[i][j]);
                            }
                }
            }

            if constexpr (PROMOTE && !MMA16) {
                const float sa_t = AMODE == FGS_SCALE_TENSOR ? p.sA[0] : 1.0f;
                const float sb_t = BMODE == FGS_SCALE_TENSOR ? sBp[0] : 1.0f;
                if constexpr (B_TILE) {
                    // columns of this lane's accumulators: n = 64*wn + 32*j + 8*q + 4*(l>>5) + e
                    const float* ssb = reinterpret_cast<const float*>(st + L::A_BYTES + L::B_BYTES);
    #pragma unroll
                    for (int j = 0; j < TJ; ++j)
    #pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 s4 = *reinterpret_cast<const float4*>(ssb + 64 * wn + 32 * j + 8 * q + 4 * (l >> 5));
                            const float sbv[4] = {s4.x, s4.y, s4.z, s4.w};
    #pragma unroll
                            for (int i = 0; i < TI; ++i) {
                                const float fa = AMODE == FGS_SCALE_TENSOR ? sa_t : sa[i];
    #pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    acc[i][j][4 * q + e] = __builtin_fmaf(part[i][j][4 * q + e], fa * sbv[e], acc[i][j][4 * q + e]);
                            }
                        }
                } else {
                    const float fb = BMODE == FGS_SCALE_TENSOR ? sb_t : sb_blk;
    #pragma unroll
                    for (int i = 0; i < TI; ++i) {
                        const float f = (AMODE == FGS_SCALE_TENSOR ? sa_t : sa[i]) * fb;
    #pragma unroll
                        for (int j = 0; j < TJ; ++j)
    #pragma unroll
                            for (int r = 0; r < 16; ++r)
                                acc[i][j][r] = __builtin_fmaf(part[i][j][r], f, acc[i][j][r]);
                    }
                }
            }
        }

        wait_lds_dma();
        __syncthreads();
    }

    if constexpr (MX && !MMA8) {
        // 2^(E_A + E_B - 254) by exponent arithmetic (exact up to FP32
        // overflow or underflow); NaN rows and columns
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int sh = (int)ea[i] + (int)eb - 254;
            const bool rnan = s_mx_nan[WM * wm + 32 * i + (l & 31)] != 0;
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int cn = 64 * wn + 32 * j + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
                    const float v = __builtin_ldexpf(acc[i][j][r], sh);
                    acc[i][j][r] = (rnan || s_mx_nan[BM + cn]) ? __builtin_nanf("") : v;
                }
        }
    } else if constexpr (!PROMOTE && !MX) {
        const float f = NV ? p.tsA[0] * p.tsB[0] : p.sA[0] * sBp[0];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] *= f;
    }

    // ------------------------------------------- E4M3 output (optional) --
    // The BF16-rounded outputs quantized in 1x128 tiles along N for the next
    // layer (the online rule of the quantizers: s = fl32(amax / 448), code =
    // E4M3_RNE(fl32(y / s))).  A tile row's 128 columns live in two waves
    // (wn, wn ^ 1), 64 in each.  Rows are taken in row sets rs of the
    // accumulator layout:
    //  32x32 tiles: rs = i, lane row 32 i + l % 32; the row's 64 columns of
    //    the wave lie in lanes l and l ^ 32, 32 values each (j, q, e);
    //  16x16 tiles (MMA16): rs = 2 i + h, lane row 32 i + 16 h + l % 16; the
    //    row's 64 columns lie in lanes l, l ^ 16, l ^ 32, l ^ 48, 16 values
    //    each (j, quarter 2 h + c, e).
    // The row maxima meet in the LDS stages, free once the K loop's last
    // barrier has passed.  Launches with q_out need N % 128 == 0.
    if constexpr (OUT_BF16 && GROUP != GROUP_K && !MMA8) {
        if (p.q_out) {
            constexpr int RS = MMA16 ? 2 * TI : TI;      // row sets per lane
            constexpr int QS = MMA16 ? 2 : 4;            // float quads per (row set, j)
            auto lane_row = [&](int rs) -> int {
                return MMA16 ? WM * wm + 32 * (rs >> 1) + 16 * (rs & 1) + (l & 15) : WM * wm + 32 * rs + (l & 31);
            };
            // float quad c (0 .. QS-1) of row set rs and sub-tile j, and its
            // first column within the tile
            auto quad = [&](int rs, int j, int c) -> float4 {
                const f32x16& a = acc[MMA16 ? rs >> 1 : rs][j];
                const int o = MMA16 ? 4 * (2 * (rs & 1) + c) : 4 * c;
                return make_float4(a[o], a[o + 1], a[o + 2], a[o + 3]);
            };
            auto quad_col = [&](int j, int c) -> int {
                return MMA16 ? 64 * wn + 32 * j + 16 * c + 4 * (l >> 4) : 64 * wn + 32 * j + 8 * c + 4 * (l >> 5);
            };
            uint32_t* rmax = reinterpret_cast<uint32_t*>(smem);      // [BM][NWN] |BF16| bits
#pragma unroll
            for (int rs = 0; rs < RS; ++rs) {
                uint32_t mx = 0;
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int c = 0; c < QS; ++c) {
                        const float4 v = quad(rs, j, c);
                        const uint32_t h01 = bf16x2_rne(v.x, v.y);
                        const uint32_t h23 = bf16x2_rne(v.z, v.w);
                        mx = max(mx, max(max(h01 & 0x7FFFu, (h01 >> 16) & 0x7FFFu),
                                         max(h23 & 0x7FFFu, (h23 >> 16) & 0x7FFFu)));
                    }
                if constexpr (MMA16) mx = max_xor16(mx);
                mx = max_xor32(mx);
                if (l < (MMA16 ? 16 : 32)) rmax[lane_row(rs) * NWN + wn] = mx;
            }
            __syncthreads();
#pragma unroll
            for (int rs = 0; rs < RS; ++rs) {
                const int r = lane_row(rs);
                const int64_t m = m0 + r;
                const E4M3Block b = e4m3_block_from_amax_bits(max(rmax[r * NWN + wn], rmax[r * NWN + (wn ^ 1)]));
                if (m < m_end) {
                    if (l < (MMA16 ? 16 : 32) && (wn & 1) == 0) p.s_out[((n0 + 64 * wn) / 128) * p.M + m] = b.s;
#pragma unroll
                    for (int j = 0; j < TJ; ++j)
#pragma unroll
                        for (int c = 0; c < QS; ++c) {
                            const float4 v = quad(rs, j, c);
                            const int64_t n = n0 + quad_col(j, c);
                            const uint32_t h01 = bf16x2_rne(v.x, v.y);
                            const uint32_t h23 = bf16x2_rne(v.z, v.w);
                            uint32_t c4 = 0x7F7F7F7Fu;
                            if (!b.nan)
                                c4 = e4m3_pack4(e4m3_quotient_bits(h01 << 16, b), e4m3_quotient_bits(h01 & 0xFFFF0000u, b),
                                                e4m3_quotient_bits(h23 << 16, b), e4m3_quotient_bits(h23 & 0xFFFF0000u, b));
                            if (n + 3 < p.N) *reinterpret_cast<uint32_t*>(p.q_out + m * p.N + n) = c4;
                        }
                }
            }
            if (!p.C) return;
        }
    }

    // ------------------------------------------ staged FP32 epilogue --
    // MoE weight gradients: most experts hold one or two 128-token blocks,
    // so a tile is mostly its 64 KiB of FP32 output.  Stored straight from
    // the accumulator layout, each store instruction writes 32 bytes to each
    // of 32 rows; through the LDS stages (free after the K loop's last
    // barrier) each instruction writes two whole 512-byte rows.  Row r of
    // the staged tile holds its 16-byte chunk c at slot c ^ (r & 31), so the
    // column-wise writes and the row-wise reads both spread over the banks.
    if constexpr (!OUT_BF16 && GROUP == GROUP_K && !MMA16) {
        static_assert(BN == 128 && 2 * L::STAGE >= BM * BN * 4, "the FP32 tile must fit the two LDS stages");
        // uniform over the workgroup: a full-width tile and 16-byte rows
        if (n0 + BN <= p.N && (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0) {
            float* st = reinterpret_cast<float*>(smem);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = WM * wm + 32 * i + (l & 31);
                        const int c = 16 * wn + 8 * j + 2 * q + (l >> 5);
                        *reinterpret_cast<float4*>(st + r * BN + 4 * (c ^ (r & 31))) =
                            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    }
            __syncthreads();
            const int c = t & 31;
            float* const Ct = static_cast<float*>(p.C) + c_off + m0 * p.ldc + n0 + 4 * c;
#pragma unroll
            for (int it = 0; it < BM / (NT / 32); ++it) {
                const int r = (NT / 32) * it + (t >> 5);
                if (m0 + r < m_end)
                    *reinterpret_cast<float4*>(Ct + r * p.ldc) =
                        *reinterpret_cast<const float4*>(st + r * BN + 4 * (c ^ (r & 31)));
            }
            return;
        }
    }

    // ------------------------------------------------------ epilogue --
    // acc[i][j] floats 4q .. 4q+3 are four consecutive columns of one row:
    // 32x32 tiles: row 32 i + l % 32, columns 32 j + 8 q + 4 (l / 32) ..;
    // 16x16 tiles (MMA16): row 32 i + 16 (q / 2) + l % 16, columns
    // 32 j + 16 (q % 2) + 4 (l / 16) ..
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t m = MMA16 ? m0 + WM * wm + 32 * i + 16 * (q >> 1) + (l & 15)
                                        : m0 + WM * wm + 32 * i + (l & 31);
                if (m >= m_end) continue;
                const int64_t n = MMA16 ? n0 + 64 * wn + 32 * j + 16 * (q & 1) + 4 * (l >> 4)
                                        : n0 + 64 * wn + 32 * j + 8 * q + 4 * (l >> 5);
                if constexpr (OUT_BF16) {
                    uint16_t* C = static_cast<uint16_t*>(p.C) + c_off + m * p.ldc + n;
                    const uint32_t h01 = bf16x2_rne(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                    const uint32_t h23 = bf16x2_rne(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    if (n + 3 < p.N && ((reinterpret_cast<uintptr_t>(C) & 7) == 0)) {
                        *reinterpret_cast<uint2*>(C) = make_uint2(h01, h23);
                    } else {
                        const uint32_t h[4] = {h01 & 0xFFFFu, h01 >> 16, h23 & 0xFFFFu, h23 >> 16};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) C[e] = (uint16_t)h[e];
                    }
                } else {
                    float* C = static_cast<float*>(p.C) + c_off + m * p.ldc + n;
                    if (n + 3 < p.N && ((reinterpret_cast<uintptr_t>(C) & 15) == 0)) {
                        *reinterpret_cast<float4*>(C) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                                    acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) C[e] = acc[i][j][4 * q + e];
                    }
                }
            }
    }
}

// MXFP8 references of the exact path: for each of the rows of A (rows
// 0 .. M-1 of out) and of B (rows M .. M+N-1), the largest E8M0 scale byte
// of the row over all of K other than the NaN byte 0xFF (0 if there is
// none), with bit 8 set when the row holds a NaN byte.  One wave per row,
// each lane reading 16 bytes at a time where the rows allow it (4 where they
// do not), the lanes' results met by lane exchange.  Formed once per launch
// instead of by every tile that reads the row (each B row is otherwise
// scanned again by every m-tile).
__global__ __launch_bounds__(256) void mx_row_ref_kernel(const uint8_t* __restrict__ sA, int64_t M,
                                                          const uint8_t* __restrict__ sB, int64_t N,
                                                          int64_t ksc, uint16_t* __restrict__ out)
{
    const int l = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= M + N) return;                                   // whole waves
    const uint8_t* const row = r < M ? sA + r * ksc : sB + (r - M) * ksc;
    uint32_t mref = 0, nan = 0;
    auto scan_word = [&](uint32_t w4) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t v = (w4 >> (8 * b)) & 0xFFu;
            nan |= v == 0xFFu;
            mref = max(mref, v == 0xFFu ? 0u : v);
        }
    };
    if ((ksc & 15) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
        const uint4* src = reinterpret_cast<const uint4*>(row);
        for (int64_t c = l; c < ksc / 16; c += 64) {
            const uint4 q = src[c];
            scan_word(q.x);
            scan_word(q.y);
            scan_word(q.z);
            scan_word(q.w);
        }
    } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(row);
        for (int64_t c = l; c < ksc / 4; c += 64) scan_word(src[c]);
    }
    mref = max_xor32(max_xor16(max_lanes16(mref)));
    nan = max_xor32(max_xor16(max_lanes16(nan)));
    if (l == 0) out[r] = (uint16_t)(mref | (nan << 8));
}

template <class S, int AMODE, int BMODE, int GROUP, int ELEMS = 0, bool MMA8 = false>
hipError_t launch_modes(GemmParams p, const GemmArgs& a, bool bf16, hipStream_t s)
{
    p.tiles_n = (int32_t)((a.N + S::BN - 1) / S::BN);
    // row groups: every group can add one partial m-tile; a launch that
    // takes only groups of at least grp_lo rows holds at most M / grp_lo of
    // them, one that takes groups below grp_hi rows at most
    // ceil((grp_hi - 1) / BM) tiles per group
    int64_t tm = (a.M + S::BM - 1) / S::BM;
    if constexpr (GROUP == GROUP_M) {
        tm += p.grp_lo > 0 ? std::min<int64_t>(a.G, a.M / p.grp_lo) : a.G;
        if (p.grp_hi < INT32_MAX) tm = std::min<int64_t>(tm, (int64_t)a.G * ((p.grp_hi - 1 + S::BM - 1) / S::BM));
    }
    p.tiles_m = (int32_t)tm;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n * (GROUP == GROUP_K ? a.G : 1);
    const dim3 grid((unsigned)tiles);
    // the E4M3-output epilogue exists for BF16 output on the exact path of
    // the row-grouped and dense schedules only; any other launch with q_out
    // would leave it unwritten, so it is refused before launching
    if (a.q_out && (!bf16 || MMA8 || GROUP == GROUP_K)) return hipErrorInvalidValue;
    if (a.name_out) {
        // the instantiation, as profilers print it without namespaces and
        // arguments
        snprintf(a.name_out, a.name_len, "gemm_block_scaled_kernel<Shape<%d, %d, %d>, %d, %d, %s, %d, %d, %s>",
                 S::NWM, S::NWN, S::TI, AMODE, BMODE, bf16 ? "true" : "false", GROUP, ELEMS, MMA8 ? "true" : "false");
        return hipSuccess;
    }
    constexpr bool a_lds = S::TI == 4 && AMODE == FGS_SCALE_TILE_1x128;   // the kernel's A_LDS
    constexpr int scw = AMODE == FGS_SCALE_MX32_E8M0 ? 1 : (AMODE == FGS_SCALE_NV16_E4M3 ? 2 : 0);   // the kernel's SCW
    const size_t lds = 2 * (size_t)Lds<S, AMODE == FGS_SCALE_NV16_E4M3 ? 64 : 128, BMODE == FGS_SCALE_TILE_1x128, a_lds,
                                       scw>::STAGE;
    auto k = bf16 ? gemm_block_scaled_kernel<S, AMODE, BMODE, true, GROUP, ELEMS, MMA8>
                  : gemm_block_scaled_kernel<S, AMODE, BMODE, false, GROUP, ELEMS, MMA8>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, dim3(64 * S::NWM * S::NWN), lds, s, p);
    return hipGetLastError();
}

// The wide tile does twice the work of the 256 x 128 one in about 1.85x its
// time on the exact path (measured on the Llama-3-8B shapes; 1.6-1.7 on
// 8192 x 28672 x 4096) and about 1.6x on the FP8 instructions (1.45-1.65 on
// that shape), but halves the tile count, so a problem whose wide tiles fill
// the last round poorly runs faster on the narrow tile: compare rounds x
// time per round.  The caller may force either tile (GemmArgs::tile).
bool prefer_wide(const GemmArgs& a)
{
    if (a.tile != FGS_TILE_AUTO) return a.tile == FGS_TILE_WIDE;
    const int64_t cus = device_cus();   // one workgroup of either dense shape fills a CU's LDS
    const int64_t tm = (a.M + ShapeWide::BM - 1) / ShapeWide::BM;
    const int64_t wide = tm * ((a.N + ShapeWide::BN - 1) / ShapeWide::BN);
    const int64_t narrow = ((a.M + ShapeDense::BM - 1) / ShapeDense::BM) * ((a.N + ShapeDense::BN - 1) / ShapeDense::BN);
    const double t_wide = (a.fp8_mma ? 1.6 : 1.85) * (double)((wide + cus - 1) / cus);
    const double t_narrow = (double)((narrow + cus - 1) / cus);
    return t_wide <= t_narrow;
}

// Modes without promotion (one scale per operand for all of K: per-tensor
// E4M3, NVFP4, and MX on the exact path) keep 128 accumulators per lane and
// can take the wide tile; the promoted modes hold partial sums too and take
// the 256 x 128 tile.  MMA8: the same modes on the FP8 matrix instructions
// (NVFP4's E4M3 block scales have no FP8-instruction form and are rejected).
template <bool MMA8>
hipError_t dispatch_dense(const GemmParams& p, const GemmArgs& a, bool bf16, hipStream_t s)
{
    using D = ShapeDense;
    using W = ShapeWide;
    constexpr int NONE = GROUP_NONE;
    const bool wide = prefer_wide(a);
    const int amode = a.A.scale_mode, bmode = a.B.scale_mode;
    // promoted modes: the 256 x 128 tile, or the 256 x 256 tile of 16x16
    // output tiles (FP8 instructions: every mode; exact path: not with 1x128
    // B scales, whose four scale factors per lane and tile would not fit in
    // registers beside the held FP16 B fragments)
    constexpr int TL = FGS_SCALE_TILE_1x128, BL = FGS_SCALE_BLOCK_128x128, TN = FGS_SCALE_TENSOR;
    auto promoted = [&](auto am, auto bm) -> hipError_t {
        constexpr int A_ = decltype(am)::value, B_ = decltype(bm)::value;
        if constexpr (MMA8 || B_ != FGS_SCALE_TILE_1x128)
            if (wide) return launch_modes<W, A_, B_, NONE, 0, MMA8>(p, a, bf16, s);
        return launch_modes<D, A_, B_, NONE, 0, MMA8>(p, a, bf16, s);
    };
    using IC_TL = std::integral_constant<int, TL>;
    using IC_BL = std::integral_constant<int, BL>;
    using IC_TN = std::integral_constant<int, TN>;
    if (amode == FGS_SCALE_TILE_1x128) {
        if (bmode == FGS_SCALE_BLOCK_128x128) return promoted(IC_TL{}, IC_BL{});
        if (bmode == FGS_SCALE_TILE_1x128) return promoted(IC_TL{}, IC_TL{});
        if (bmode == FGS_SCALE_TENSOR) return promoted(IC_TL{}, IC_TN{});
    } else if (amode == FGS_SCALE_MX32_E8M0 && bmode == FGS_SCALE_MX32_E8M0) {
        if (wide) return launch_modes<W, FGS_SCALE_MX32_E8M0, FGS_SCALE_MX32_E8M0, NONE, 0, MMA8>(p, a, bf16, s);
        return launch_modes<D, FGS_SCALE_MX32_E8M0, FGS_SCALE_MX32_E8M0, NONE, 0, MMA8>(p, a, bf16, s);
    } else if (amode == FGS_SCALE_NV16_E4M3 && bmode == FGS_SCALE_NV16_E4M3) {
        if constexpr (!MMA8) {
            if (wide) return launch_modes<W, FGS_SCALE_NV16_E4M3, FGS_SCALE_NV16_E4M3, NONE>(p, a, bf16, s);
            return launch_modes<D, FGS_SCALE_NV16_E4M3, FGS_SCALE_NV16_E4M3, NONE>(p, a, bf16, s);
        }
    } else if (amode == FGS_SCALE_TENSOR) {
        if (bmode == FGS_SCALE_TENSOR) {
            const int elems = (a.A.elem == FGS_ELEM_E5M2 ? 1 : 0) | (a.B.elem == FGS_ELEM_E5M2 ? 2 : 0);
            constexpr int T = FGS_SCALE_TENSOR;
            switch (elems) {
            case 1:
                if (wide) return launch_modes<W, T, T, NONE, 1, MMA8>(p, a, bf16, s);
                return launch_modes<D, T, T, NONE, 1, MMA8>(p, a, bf16, s);
            case 2:
                if (wide) return launch_modes<W, T, T, NONE, 2, MMA8>(p, a, bf16, s);
                return launch_modes<D, T, T, NONE, 2, MMA8>(p, a, bf16, s);
            case 3:
                if (wide) return launch_modes<W, T, T, NONE, 3, MMA8>(p, a, bf16, s);
                return launch_modes<D, T, T, NONE, 3, MMA8>(p, a, bf16, s);
            default:
                if (wide) return launch_modes<W, T, T, NONE, 0, MMA8>(p, a, bf16, s);
                return launch_modes<D, T, T, NONE, 0, MMA8>(p, a, bf16, s);
            }
        }
        if (bmode == FGS_SCALE_BLOCK_128x128) return promoted(IC_TN{}, IC_BL{});
        if (bmode == FGS_SCALE_TILE_1x128) return promoted(IC_TN{}, IC_TL{});
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_gemm_fp8(const GemmArgs& a, hipStream_t stream)
{
    GemmParams p{};
    p.A = static_cast<const uint8_t*>(a.A.data);
    p.B = static_cast<const uint8_t*>(a.B.data);
    p.sA = static_cast<const float*>(a.A.scales);
    p.sB = static_cast<const float*>(a.B.scales);
    const bool nv = a.A.elem == FGS_ELEM_E2M1;
    p.lda = nv ? a.A.ld / 2 : a.A.ld;
    p.ldb = nv ? a.B.ld / 2 : a.B.ld;
    p.tsA = a.A.tensor_scale;
    p.tsB = a.B.tensor_scale;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.C = a.C;
    p.ldc = a.ldc;
    p.offsets = a.group_offsets;
    p.G = a.G;
    p.T = a.T;
    p.q_out = a.q_out;
    p.s_out = a.s_out;
    p.grp_lo = 0;
    p.grp_hi = INT32_MAX;
    if (a.M == 0 || a.N == 0) return hipSuccess;
    const bool bf16 = a.out_bf16 != 0;
    if (a.fp8_mma && a.q_out) return hipErrorInvalidValue;   // no E4M3-output epilogue on the FP8 instructions
    if (a.group_k) {
        if (a.G == 0) return hipSuccess;
        // 128 x 128 tiles, two workgroups per CU: most experts hold one or
        // two 128-token blocks, so each tile is mostly its 64 KiB of FP32
        // output, and two resident workgroups overlap one's stores with the
        // other's loads and MFMAs (1.4x the 256 x 128 tile on DeepSeek-V3)
        if (a.A.scale_mode == FGS_SCALE_TILE_1x128 && a.B.scale_mode == FGS_SCALE_TILE_1x128) {
            if (a.fp8_mma)
                return launch_modes<ShapeGrouped, FGS_SCALE_TILE_1x128, FGS_SCALE_TILE_1x128, GROUP_K, 0, true>(p, a, bf16, stream);
            return launch_modes<ShapeGrouped, FGS_SCALE_TILE_1x128, FGS_SCALE_TILE_1x128, GROUP_K>(p, a, bf16, stream);
        }
        return hipErrorInvalidValue;
    }
    if (a.group_offsets) {
        p.b_group_stride = a.N * a.B.ld;
        p.sb_group_stride = ((a.N + 127) / 128) * (a.K / BK);
        if (a.A.scale_mode == FGS_SCALE_TILE_1x128 && a.B.scale_mode == FGS_SCALE_BLOCK_128x128) {
            // Groups of at least kWideRows rows take the 256 x 256 tile with
            // 16x16 output tiles, groups below kShortRows the 64 x 128 tile
            // (three workgroups per CU keep more weight bytes in flight for
            // the groups that only stream weights), the rest the 128 x 128
            // tile: three launches on the stream, each one's device schedule
            // skipping the others' groups.  Measured per tile: long groups 1.11-1.16 PF
            // on the 256 x 256 tile against 0.93-0.98 on the 128 x 128 one;
            // groups of 16-64 rows stream their weights at 4.0-4.3 TB/s on
            // the 128 x 128 tile, 3.3-3.4 on the 256 x 256 one.
            // The FP8 matrix instructions take the same split.
            GemmParams pt = p, ps = p, pl = p;
            pt.grp_hi = kShortRows;
            ps.grp_lo = kShortRows;
            ps.grp_hi = kWideRows;
            pl.grp_lo = kWideRows;
            auto split = [&](auto mma8) -> hipError_t {
                constexpr bool M8 = decltype(mma8)::value;
                hipError_t e = launch_modes<ShapeShort, FGS_SCALE_TILE_1x128, FGS_SCALE_BLOCK_128x128, GROUP_M, 0, M8>(pt, a, bf16, stream);
                if (e != hipSuccess) return e;
                e = launch_modes<ShapeGrouped, FGS_SCALE_TILE_1x128, FGS_SCALE_BLOCK_128x128, GROUP_M, 0, M8>(ps, a, bf16, stream);
                if (e != hipSuccess) return e;
                return launch_modes<ShapeWide, FGS_SCALE_TILE_1x128, FGS_SCALE_BLOCK_128x128, GROUP_M, 0, M8>(pl, a, bf16, stream);
            };
            return a.fp8_mma ? split(std::true_type{}) : split(std::false_type{});
        }
        return hipErrorInvalidValue;
    }
    if (a.fp8_mma) return dispatch_dense<true>(p, a, bf16, stream);
    if (a.A.scale_mode == FGS_SCALE_MX32_E8M0 && a.workspace && !a.name_out) {
        // the rows' reference bytes, once, into the caller's workspace
        const int64_t rows = a.M + a.N;
        uint16_t* ref = static_cast<uint16_t*>(a.workspace);
        hipLaunchKernelGGL(mx_row_ref_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                           reinterpret_cast<const uint8_t*>(a.A.scales), a.M, reinterpret_cast<const uint8_t*>(a.B.scales),
                           a.N, a.K / 32, ref);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.mx_ref = ref;
    }
    return dispatch_dense<false>(p, a, bf16, stream);
}

// MXFP8 and NVFP4 operands take the same kernel (decode and scale handling
// selected by the scale mode).
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t stream)
{
    return launch_gemm_fp8(a, stream);
}

hipError_t launch_gemm_nvfp4(const GemmArgs& a, hipStream_t stream)
{
    return launch_gemm_fp8(a, stream);
}

} // namespace fgs
