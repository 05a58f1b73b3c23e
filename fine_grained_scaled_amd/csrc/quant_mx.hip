// quant_mx.hip -- MXFP8 quantization on gfx950: E4M3 codes with one E8M0
// power-of-two scale per 32 contiguous elements.
//
// "Accelerating FP8 training performance with the NVIDIA NeMo framework":
// MXFP8 scales blocks of 32 values.  The scale rule (the power-of-two
// counterpart of amax / 448): 2^e with e the smallest integer such that
// amax <= 448 * 2^e, clamped to [-127, 127]; the scale byte is e + 127 and
// code = E4M3_RNE_SAT(x * 2^-e) (the multiply is exact).  A block holding
// NaN/Inf gets scale byte 0xFF and NaN codes; an all-zero block gets e = 0.
//
// With amax = f * 2^E (1 <= f < 2): f <= 1.75 needs e = E - 8 (448 = 1.75 *
// 2^8), f > 1.75 needs e = E - 7; on BF16 bits f > 1.75 is "mantissa field
// > 0x60".  A subnormal amax (< 2^-126) always clamps to e = -127.
//
// One workgroup (256 threads, 4 waves) owns a 128 x 128 block of the BF16
// source; thread t (wave w, lane l) holds the 8 x 8 sub-block with columns
// c0 + 8*(l & 15) .. +7 and rows r0 + 8*(4w + (l >> 4)) .. +7.  A row-wise
// 32-element block spans the 4 lanes of a DPP quad; a column-wise block
// (32 rows) is exactly one wave's rows, reduced across its four 16-lane
// rows.  Column-wise codes are transposed through LDS so every store of qT
// is a full 128-byte row.
#include "fgs_device.h"
#include "fgs_internal.h"

namespace fgs {

namespace {

constexpr int TB = 128;
constexpr int TPAD = 16;

__device__ __forceinline__ uint32_t abs_max8(const uint4& v)
{
    uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
    uint32_t c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
    uint32_t m0 = max(a & 0xFFFFu, a >> 16), m1 = max(b & 0xFFFFu, b >> 16);
    uint32_t m2 = max(c & 0xFFFFu, c >> 16), m3 = max(d & 0xFFFFu, d >> 16);
    return max(max(m0, m1), max(m2, m3));
}

__device__ __forceinline__ uint32_t raw_elem(const uint4& v, int j)
{
    uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// E8M0 block parameters from the block amax given as |BF16| bits.
struct MXBlock {
    uint32_t code;   // scale byte e + 127 (0xFF for a non-finite block)
    float inv;       // 2^-e
    bool nan;
};

__device__ __forceinline__ MXBlock mx_block(uint32_t amax16)
{
    MXBlock b;
    b.nan = amax16 >= 0x7F80u;
    if (b.nan) {
        b.code = 0xFFu;
        b.inv = 1.0f;
        return b;
    }
    int e;
    if (amax16 == 0) {
        e = 0;
    } else {
        const int ef = (int)(amax16 >> 7);
        e = ef - 135 + ((amax16 & 0x7Fu) > 0x60u ? 1 : 0);
        if (ef == 0 || e < -127) e = -127;
    }
    b.code = (uint32_t)(e + 127);
    b.inv = as_f32((uint32_t)(127 - e) << 23);
    return b;
}

// Codes of eight BF16 values (raw 16-bit patterns) of one block.  x * 2^-e
// is exact and lies in [-448, 448] (e is the smallest exponent with
// amax <= 448 * 2^e; a clamp at e = -127 only shrinks |x * 2^-e|), where
// the hardware converter equals the saturating RNE encoder with the sign of
// the input (see e4m3_pack4).  A non-finite block takes 0x7F codes.
__device__ __forceinline__ uint2 mx_code8(const uint32_t h[8], const MXBlock& b)
{
    if (b.nan) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = as_f32(h[j] << 16) * b.inv;
    return make_uint2(e4m3_pack4(y[0], y[1], y[2], y[3]), e4m3_pack4(y[4], y[5], y[6], y[7]));
}

__global__ __launch_bounds__(256) void quant_mx_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ qT, uint8_t* __restrict__ scalesT)
{
    __shared__ __align__(16) uint8_t tbuf[TB][TB + TPAD];

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = l & 15, rg = 4 * w + (l >> 4);
    const int64_t r0 = (int64_t)blockIdx.y * TB, c0 = (int64_t)blockIdx.x * TB;
    const int64_t col = c0 + 8 * cg;
    const bool col_ok = col < cols;

    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t row = r0 + 8 * rg + u;
        if (col_ok && row < rows)
            v[u] = load_nt16(x + row * ldx + col);
        else
            v[u] = make_uint4(0, 0, 0, 0);
    }

    // ---------------- row-wise: 32-element blocks along columns --------
    if (q) {
        const int64_t nsc = cols / 32;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const MXBlock b = mx_block(max_lanes4(abs_max8(v[u])));
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = raw_elem(v[u], j);
            const uint2 codes = mx_code8(h, b);
            const int64_t row = r0 + 8 * rg + u;
            if (col_ok && row < rows) {
                store_nt8(q + row * cols + col, codes);
                if ((cg & 3) == 0) scales[row * nsc + col / 32] = (uint8_t)b.code;
            }
        }
    }

    // ---------------- column-wise: 32-row blocks along rows -------------
    if (qT) {
        const int64_t nscT = rows / 32;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t m = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) m = max(m, raw_elem(v[u], j) & 0x7FFFu);
            m = max_xor32(max_xor16(m));
            const MXBlock b = mx_block(m);
            uint32_t h[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = raw_elem(v[u], j);
            *reinterpret_cast<uint2*>(&tbuf[8 * cg + j][8 * rg]) = mx_code8(h, b);
            if ((l >> 4) == 0 && col_ok) scalesT[(col + j) * nscT + r0 / 32 + w] = (uint8_t)b.code;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int trow = 32 * i + (t >> 3), chunk = t & 7;
            const int64_t orow = c0 + trow;
            if (orow < cols) {
                const uint4 d = *reinterpret_cast<const uint4*>(&tbuf[trow][16 * chunk]);
                store_nt16(qT + orow * rows + r0 + 16 * chunk, d);
            }
        }
    }
}

} // namespace

hipError_t launch_quant_mx(const QuantMXArgs& a, hipStream_t stream)
{
    const int64_t nbr = (a.rows + TB - 1) / TB, nbc = (a.cols + TB - 1) / TB;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_mx_kernel, dim3((unsigned)nbc, (unsigned)nbr), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.x), a.rows, a.cols, a.ldx, a.q, a.scales, a.qT, a.scalesT);
    return hipGetLastError();
}

} // namespace fgs
