// fgs_device.h -- device helpers of the gfx950 kernels (internal header of
// libfgs; never included by host-only code outside csrc/).
//
// Arithmetic rules the kernels must reproduce bit for bit:
//  * FP32-scaled E4M3 ("Can you explain the role of FP8 precision in
//    DeepSeek-V3 training", sections "Fine-grained quantization", "Online
//    quantization"): s = fl32(amax / 448), code = E4M3_RNE_SAT(fl32(x / s)).
//  * Everything is IEEE binary32 with round-to-nearest-even; the library is
//    compiled with -ffp-contract=off so every fused multiply-add below is
//    written out on purpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgs {

// ------------------------------------------------------------------------
// bit casts
// ------------------------------------------------------------------------
__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// BF16 pair packed in a 32-bit word -> its two FP32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }

// 16 bytes read once with the non-temporal hint (global_load_dwordx4 ... nt):
// streamed inputs are not kept in the caches for reuse that never comes.
__device__ __forceinline__ uint4 load_nt16(const void* p)
{
    const uint32_t* q = static_cast<const uint32_t*>(p);
    return make_uint4(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                      __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3));
}

// 8 and 16 bytes written with the non-temporal hint: streamed outputs.
__device__ __forceinline__ void store_nt8(void* p, const uint2& v)
{
    uint32_t* q = static_cast<uint32_t*>(p);
    __builtin_nontemporal_store(v.x, q);
    __builtin_nontemporal_store(v.y, q + 1);
}
__device__ __forceinline__ void store_nt16(void* p, const uint4& v)
{
    uint32_t* q = static_cast<uint32_t*>(p);
    __builtin_nontemporal_store(v.x, q);
    __builtin_nontemporal_store(v.y, q + 1);
    __builtin_nontemporal_store(v.z, q + 2);
    __builtin_nontemporal_store(v.w, q + 3);
}

// ------------------------------------------------------------------------
// cross-lane max of non-negative integers (amax carried as |BF16| bits,
// where the integer order equals the value order and NaN > Inf > finite,
// so the maximum propagates NaN exactly and independently of order).
// ------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, CTRL, 0xF, 0xF, false);
    return v > o ? v : o;
}
// quad_perm [1,0,3,2] = xor 1; [2,3,0,1] = xor 2; row_half_mirror; row_mirror
constexpr int DPP_XOR1 = 0xB1;
constexpr int DPP_XOR2 = 0x4E;
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// max over aligned groups of 2 / 4 / 16 lanes (every lane gets the result)
__device__ __forceinline__ uint32_t max_lanes2(uint32_t v) { return dpp_max<DPP_XOR1>(v); }
__device__ __forceinline__ uint32_t max_lanes4(uint32_t v)
{
    return dpp_max<DPP_XOR2>(dpp_max<DPP_XOR1>(v));
}
__device__ __forceinline__ uint32_t max_lanes16(uint32_t v)
{
    v = max_lanes4(v);
    v = dpp_max<DPP_HALF_MIRROR>(v);
    return dpp_max<DPP_MIRROR>(v);
}
// max across lanes l, l^16, l^32, l^48 (the four 16-lane rows of a wave)
__device__ __forceinline__ uint32_t max_xor16(uint32_t v)
{
    uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
    return v > o ? v : o;
}
__device__ __forceinline__ uint32_t max_xor32(uint32_t v)
{
    uint32_t o = (uint32_t)__shfl_xor((int)v, 32);
    return v > o ? v : o;
}

// ------------------------------------------------------------------------
// E4M3 (OCP E4M3FN) round-to-nearest-even with saturation, for a
// non-negative finite FP32 value; returns the 7-bit magnitude code.
// ------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_code_abs(float a)
{
    // below 2^-6 the E4M3 grid is uniform with step 2^-9: round a * 2^9
    // (exact scaling) to the nearest even integer, 0..8 (8 = 2^-6, code 0x08)
    uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
    // normal range: drop 20 of the 23 mantissa bits with RNE, then rebias the
    // exponent from 127 to 7 (a carry out of the mantissa bumps the exponent)
    uint32_t b = as_u32(a);
    uint32_t nrm = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    uint32_t c = (a < 0.015625f) ? sub : nrm;
    return c < 0x7Eu ? c : 0x7Eu;
}

// ------------------------------------------------------------------------
// fl32(x / s) from a per-block reciprocal r = RN(1/s): q0 = x*r, residual
// e = q0*s - x (exact with FMA), one correction step q0 - e*r.  The signs
// work out for either sign of x, -0 included (-0 gives q0 = -0, e = +0 and
// -0 + -0 = -0).  For s = fl32(amax/448) of a BF16 amax >= 2^-64 and every
// BF16 x with |x| <= amax, of either sign (all 1.07e9 pairs, checked on the
// host), the result is IEEE x / s except for tiny x whose quotient lies
// below 2^-40, far under the first E4M3 rounding point 2^-10, so every code
// is that of the correctly rounded quotient.  Blocks with 0 < amax < 2^-64
// are pre-scaled by 2^64 on both sides, which leaves the quotient unchanged.
// ------------------------------------------------------------------------
__device__ __forceinline__ float div_by_scale(float x, float s, float r)
{
    const float q0 = x * r;
    const float e = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-e, r, q0);
}

// fl32(amax / 448) for a BF16-valued amax, by multiplication and one FMA
// correction (bit-equal to IEEE division for every BF16 amax).
__device__ __forceinline__ float scale_from_amax_448(float amax)
{
    const float inv448 = 1.0f / 448.0f;   // RN(1/448), folded at compile time
    float s0 = amax * inv448;
    float e = __builtin_fmaf(-s0, 448.0f, amax);
    return __builtin_fmaf(e, inv448, s0);
}

// RN(1 / d) for the divisors d of the E4M3 block rule (d = fl32(amax / 448)
// of a finite BF16 amax > 0, times 2^64 when amax < 2^-64, or 1): the
// hardware reciprocal (within 1 ulp) and one Newton step.  Equal to IEEE
// division for all 32639 such divisors (checked on gfx950); 1 and the other
// powers of two come out exact.
__device__ __forceinline__ float e4m3_scale_recip(float d)
{
    const float r0 = __builtin_amdgcn_rcpf(d);
    const float e = __builtin_fmaf(-d, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

// Per-block quantization constants of the FP32-scaled E4M3 rule.
struct E4M3Block {
    float s;      // the block scale written out
    float k;      // 1 or 2^64 (pre-scale of tiny blocks)
    float sp;     // s * k
    float r;      // RN(1 / sp)
    bool nan;     // amax non-finite: scale NaN, all codes 0x7F
};

// 0 < amax < 2^-64 (BF16 bits of 2^-64: 0x1F80): the pre-scaled blocks
__device__ __forceinline__ bool e4m3_block_prescaled(uint32_t amax_bits16)
{
    return amax_bits16 - 1u < 0x1F7Fu;
}

// The block takes the NaN path or the pre-scale: true exactly when
// e4m3_block_from_amax_bits gives nan or k != 1.
__device__ __forceinline__ bool e4m3_block_special(uint32_t amax_bits16)
{
    return amax_bits16 >= 0x7F80u || e4m3_block_prescaled(amax_bits16);
}

__device__ __forceinline__ E4M3Block e4m3_block_from_amax_bits(uint32_t amax_bits16)
{
    E4M3Block b;
    float amax = as_f32(amax_bits16 << 16);
    b.nan = amax_bits16 >= 0x7F80u;
    if (b.nan) {
        b.s = __builtin_nanf("");
        b.k = 1.0f; b.sp = 1.0f; b.r = 1.0f;
        return b;
    }
    b.s = (amax_bits16 == 0) ? 1.0f : scale_from_amax_448(amax);
    // an all-zero block takes k = 1: every quotient of it is a signed zero
    // with or without the pre-scale
    b.k = e4m3_block_prescaled(amax_bits16) ? 0x1p64f : 1.0f;
    b.sp = b.s * b.k;
    b.r = e4m3_scale_recip(b.sp);
    return b;
}

// The same constants for a block that e4m3_block_special rejects (finite,
// not pre-scaled): no NaN or pre-scale selects.
__device__ __forceinline__ E4M3Block e4m3_block_plain(uint32_t amax_bits16)
{
    E4M3Block b;
    b.nan = false;
    b.s = (amax_bits16 == 0) ? 1.0f : scale_from_amax_448(as_f32(amax_bits16 << 16));
    b.k = 1.0f;
    b.sp = b.s;
    b.r = e4m3_scale_recip(b.sp);
    return b;
}

// E4M3 codes of four FP32 values, packed little-endian into one word, by
// the hardware converter v_cvt_pk_fp8_f32 (round to nearest even, OCP
// E4M3).  On [-449, 449] it equals the saturating encoder above with the sign
// of the input (checked exhaustively over every FP32 bit pattern in that
// range on gfx950), and every quotient x / s of a finite block lies there:
// |x| <= amax and s = fl32(amax / 448) give |x / s| <= 448 (1 + 2^-23).
// NaN never reaches it (a block holding a NaN or Inf takes the all-0x7F
// path).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d)
{
    // the first conversion writes the low half of a word whose high half the
    // second one overwrites, so its old value is free: a's own bits, which
    // die here, save a register move of zero
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)as_u32(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// fl32(x / s) of a block element given as FP32 bits (sign kept, -0
// included).  Blocks with 0 < amax < 2^-64 (b.k != 1) take the pre-scaled
// form (x * 2^64 is exact), a branch that real data does not enter.
__device__ __forceinline__ float e4m3_quotient_bits(uint32_t xb, const E4M3Block& b)
{
    float x = as_f32(xb);
    if (__builtin_expect(b.k != 1.0f, 0)) x *= b.k;
    return div_by_scale(x, b.sp, b.r);
}

// The same quotient for a block with k == 1 and no NaN (the caller has
// ruled out both, e.g. with e4m3_block_special over the whole wave).
__device__ __forceinline__ float e4m3_quotient_plain(uint32_t xb, const E4M3Block& b)
{
    return div_by_scale(as_f32(xb), b.sp, b.r);
}

} // namespace fgs
