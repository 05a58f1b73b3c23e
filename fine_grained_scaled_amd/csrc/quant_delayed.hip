// quant_delayed.hip -- per-tensor delayed scaling to E4M3 or E5M2 on gfx950.
//
// "Can you explain the role of FP8 precision in DeepSeek-V3 training",
// section "Online quantization": online scales replace delayed ones, which
// come from the maxima of earlier steps; section "Unified E4M3 format":
// earlier frameworks used E4M3 forward and E5M2 backward.  The pages give
// neither formula; the rule built here: the scale is s = fl32(hmax / fmax)
// with hmax the NaN-propagating max of the caller's amax history (s = 1 for
// an all-zero history, NaN for a non-finite one) and fmax = 448 (E4M3) or
// 57344 (E5M2); every element is code = ENC_RNE_SAT(fl32(x / s)) (values
// past this step's range saturate, NaN gives 0x7F); this tensor's amax is
// recorded into the history slot the caller names.
//
// Because the scale is known before the data is read, one pass over x
// suffices (current per-tensor scaling needs an amax pass first): the amax
// for later steps is reduced in the same pass, one atomic per workgroup.
//
// Two kernels on the stream: delayed_scale_kernel (one workgroup) reads the
// history, writes the scale and clears the slot; quant_delayed_kernel casts
// 128 x 128 blocks (the thread layout of the E4M3 quantizer: 8 x 8 values
// per thread, 16 lanes over one 256-byte row segment) and atomically maxes
// the block amax into the slot.
#include <algorithm>

#include "fgs_device.h"
#include "fgs_internal.h"

namespace fgs {

namespace {

constexpr int TB = 128;
constexpr int TPAD = 16;

__device__ __forceinline__ uint32_t abs_max8_bf16(const uint4& v)
{
    const uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0xFFFFu, w[i] >> 16));
    return m;
}

// FP32 bit pattern of element j (0..7) of an 8-element BF16 vector (exact)
__device__ __forceinline__ uint32_t bf16_elem_bits(const uint4& v, int j)
{
    const uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
    return (j & 1) ? (w & 0xFFFF0000u) : (w << 16);
}

// E5M2 magnitude code of a non-negative FP32 value a <= 57344, round to
// nearest even.  Below 2^-14 the grid is uniform with step 2^-16 (round
// a * 2^16, an exact scaling, to the nearest even integer 0..4; 4 is the
// code of 2^-14).  Above, drop 21 of the 23 mantissa bits with RNE and
// rebias the exponent from 127 to 15 (a carry out of the mantissa bumps the
// exponent).
__device__ __forceinline__ uint32_t e5m2_code_abs(float a)
{
    const uint32_t sub = (uint32_t)__builtin_rintf(a * 65536.0f);
    const uint32_t b = as_u32(a);
    const uint32_t nrm = ((b + 0xFFFFFu + ((b >> 21) & 1u)) >> 21) - (112u << 2);
    const uint32_t c = (a < 0x1p-14f) ? sub : nrm;
    return c < 0x7Bu ? c : 0x7Bu;
}

// Four E5M2 codes by the hardware converter v_cvt_pk_bf8_f32 (OCP E5M2 on
// gfx950, round to nearest even), a in the lowest byte.  For every FP32
// magnitude in [0, 57344], of either sign, it equals e5m2_code_abs with the
// sign bit put back (checked exhaustively on gfx950), so after a clamp to
// +-57344 it is the saturating encoder.  The first conversion's old value
// is overwritten by the second, so a's own bits serve.
__device__ __forceinline__ uint32_t e5m2_pack4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)as_u32(a), false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Code of one element (FP32 bits of a BF16 value) under scale s.  The
// quotient is the IEEE FP32 division: unlike the online scales, s need not
// come from this tensor's amax, so the quotient may lie anywhere.
template <bool E5M2>
__device__ __forceinline__ uint32_t delayed_code(uint32_t xb, float s)
{
    const float y = as_f32(xb) / s;
    if (y != y) return 0x7Fu;                          // NaN x, or a NaN / zero scale
    const uint32_t sign = (as_u32(y) >> 24) & 0x80u;
    const float a = __builtin_fminf(__builtin_fabsf(y), E5M2 ? 57344.0f : 448.0f);
    return sign | (E5M2 ? e5m2_code_abs(a) : e4m3_code_abs(a));
}

template <bool E5M2>
__device__ __forceinline__ uint2 delayed_code8(const uint32_t xb[8], float s)
{
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = delayed_code<E5M2>(xb[j], s);
    return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                      c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// The same codes for finite x and a scale in [2^-60, 2^60], without the
// per-element IEEE division.  x is first clamped to +-t, t = fl32(2 fmax s):
// a quotient beyond the clamp saturates either way, and within it the
// quotient stays far from overflow.  The quotient is Markstein's correction
// from r = RN(1/s): q0 = x r, e = q0 s - x (exact), q = q0 - e r.  For every
// BF16 significand of x and every FP32 significand of s (all 2^31 pairs with
// sign, x and s in [1, 2), checked on the host) it equals IEEE x / s, and
// each step is exact under scaling by powers of two while its operands and
// results stay normal.  They do wherever the code can differ from 0: there
// |q| >= 2^-17 and s >= 2^-60, so |x| >= 2^-77 and the residual is exact.
// The sign of x, -0 included, carries through the correction.
template <bool E5M2>
__device__ __forceinline__ uint2 delayed_code8_fast(const uint32_t xb[8], float s, float r, float t)
{
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float x = __builtin_amdgcn_fmed3f(as_f32(xb[j]), -t, t);
        const float q0 = x * r;
        const float e = __builtin_fmaf(q0, s, -x);
        y[j] = __builtin_fmaf(-e, r, q0);
    }
    if constexpr (E5M2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = __builtin_amdgcn_fmed3f(y[j], -57344.0f, 57344.0f);
        return make_uint2(e5m2_pack4(y[0], y[1], y[2], y[3]), e5m2_pack4(y[4], y[5], y[6], y[7]));
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = __builtin_amdgcn_fmed3f(y[j], -448.0f, 448.0f);
        return make_uint2(e4m3_pack4(y[0], y[1], y[2], y[3]), e4m3_pack4(y[4], y[5], y[6], y[7]));
    }
}

// One workgroup: s from the history, then the slot is cleared for this
// step's amax (after every thread has read the history).
__global__ __launch_bounds__(256) void delayed_scale_kernel(float* __restrict__ hist, int32_t H, int32_t slot,
                                                            float fmax, float* __restrict__ scale)
{
    __shared__ uint32_t red[4];
    const int t = threadIdx.x;
    uint32_t m = 0;
    for (int i = t; i < H; i += 256) m = max(m, as_u32(hist[i]) & 0x7FFFFFFFu);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    if (t == 0) {
        m = max(max(red[0], red[1]), max(red[2], red[3]));
        float s;
        if (m >= 0x7F800000u)
            s = __builtin_nanf("");
        else if (m == 0)
            s = 1.0f;
        else
            s = as_f32(m) / fmax;
        scale[0] = s;
        hist[slot] = 0.0f;
    }
}

// Workgroup (blockIdx.x, blockIdx.y) quantizes column tiles
// blockIdx.x * tpw .. + tpw - 1 of row tile blockIdx.y (up to 32), one after another,
// and adds its amax to the history slot with one atomic: same-address
// atomics are served one at a time (measured on the Llama-3-8B hybrid step,
// one per 128 x 128 tile: 15-25% of these kernels' time).  Addresses are a
// tile's uniform base plus per-lane offsets below 2^31 (Off = int32_t when
// 128 rows of every array fit, which the host checks), so the loop keeps
// few per-lane registers live.
template <bool E5M2, typename Off>
__global__ __launch_bounds__(256, 4) void quant_delayed_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    const float* __restrict__ scale, uint32_t* __restrict__ amax_slot,
    uint8_t* __restrict__ q, uint8_t* __restrict__ qT, int tpw)
{
    __shared__ uint32_t red[4];
    __shared__ __align__(16) uint8_t tbuf[TB][TB + TPAD];

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = l & 15, rg = 4 * w + (l >> 4);
    const int64_t r0 = (int64_t)blockIdx.y * TB;
    const int64_t nbc = (cols + TB - 1) / TB;
    const float s = scale[0];
    const int lrow = 8 * rg;           // the thread's first row of the tile
    uint32_t mrun = 0;                 // the wave's amax over its tiles

    for (int k = 0; k < tpw; ++k) {
        const int64_t cb = (int64_t)blockIdx.x * tpw + k;
        if (cb >= nbc) break;                         // uniform
        const int64_t c0 = cb * TB;
        const bool col_ok = c0 + 8 * cg < cols;
        const uint16_t* const xt = x + r0 * ldx + c0;

        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = (col_ok && r0 + lrow + u < rows) ? load_nt16(xt + ((Off)(lrow + u) * (Off)ldx + 8 * cg))
                                                    : make_uint4(0, 0, 0, 0);

        // amax of the tile (|BF16| bits order like the values, NaN on top)
        uint32_t m = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = max(m, abs_max8_bf16(v[u]));
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
        mrun = max(mrun, m);

        // the codes of the thread's 8 x 8 values, computed once: row u is
        // c[u] (byte j = column j); the column-wise output is their byte
        // transpose.  m is the wave's amax: the branch is uniform across it.
        uint2 c[8];
        if (s >= 0x1p-60f && s <= 0x1p60f && m < 0x7F80u) {
            const float r = 1.0f / s;                        // IEEE division, once
            const float tt = (E5M2 ? 2.0f * 57344.0f : 2.0f * 448.0f) * s;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                uint32_t xb[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) xb[j] = bf16_elem_bits(v[u], j);
                c[u] = delayed_code8_fast<E5M2>(xb, s, r, tt);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                uint32_t xb[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) xb[j] = bf16_elem_bits(v[u], j);
                c[u] = delayed_code8<E5M2>(xb, s);
            }
        }
        if (q) {
            uint8_t* const qt = q + r0 * cols + c0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (col_ok && r0 + lrow + u < rows)
                    *reinterpret_cast<uint2*>(qt + ((Off)(lrow + u) * (Off)cols + 8 * cg)) = c[u];
        }
        if (qT) {
            // column j, rows 8*rg .. 8*rg+7 -> 8 contiguous bytes of qT
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t b[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) b[u] = (((j < 4) ? c[u].x : c[u].y) >> (8 * (j & 3))) & 0xFFu;
                *reinterpret_cast<uint2*>(&tbuf[8 * cg + j][lrow]) =
                    make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
            }
            __syncthreads();
            uint8_t* const qTt = qT + c0 * rows + r0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int trow = 32 * i + (t >> 3), chunk = t & 7;
                if (c0 + trow < cols) {
                    const uint4 d = *reinterpret_cast<const uint4*>(&tbuf[trow][16 * chunk]);
                    *reinterpret_cast<uint4*>(qTt + ((Off)trow * (Off)rows + 16 * chunk)) = d;
                }
            }
            __syncthreads();                          // tbuf is written again by the next tile
        }
    }
    if (l == 0) red[w] = mrun;
    __syncthreads();
    if (t == 0) {
        const uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
        atomicMax(amax_slot, m << 16);               // FP32 bits of the BF16 amax
    }
}

} // namespace

hipError_t launch_quant_delayed(const QuantDelayedArgs& a, hipStream_t stream)
{
    const bool e5 = a.elem == FGS_ELEM_E5M2;
    hipLaunchKernelGGL(delayed_scale_kernel, dim3(1), dim3(256), 0, stream,
                       a.history, a.history_len, a.slot, e5 ? 57344.0f : 448.0f, a.scale);
    const int64_t nbr = (a.rows + TB - 1) / TB, nbc = (a.cols + TB - 1) / TB;
    if (nbr > 0 && nbc > 0) {
        // 32-bit offsets when 128 rows of every array stay below 2^31
        // elements (bytes for the codes); then tiles per workgroup for about
        // two workgroups per CU in all, at most 32 (hybrid step, same box:
        // 734 us with this, 763 with eight workgroups per CU, 802 with eight
        // per CU and at most 8 tiles)
        const bool small = (int64_t)TB * std::max({a.ldx, a.cols, a.rows}) < ((int64_t)1 << 31);
        int64_t tpw = small ? nbr * nbc / (2 * (int64_t)device_cus()) : 1;
        tpw = std::max<int64_t>(1, std::min<int64_t>({tpw, 32, nbc}));
        const dim3 grid((unsigned)((nbc + tpw - 1) / tpw), (unsigned)nbr);
        const uint16_t* x = static_cast<const uint16_t*>(a.x);
        uint32_t* slot = reinterpret_cast<uint32_t*>(a.history + a.slot);
        auto k = e5 ? (small ? quant_delayed_kernel<true, int32_t> : quant_delayed_kernel<true, int64_t>)
                    : (small ? quant_delayed_kernel<false, int32_t> : quant_delayed_kernel<false, int64_t>);
        hipLaunchKernelGGL(k, grid, dim3(256), 0, stream, x, a.rows, a.cols, a.ldx, a.scale, slot, a.q, a.qT, (int)tpw);
    }
    return hipGetLastError();
}

} // namespace fgs
