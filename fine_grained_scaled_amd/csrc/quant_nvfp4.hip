// quant_nvfp4.hip -- NVFP4 quantization on gfx950: E2M1 codes (two per
// byte), one E4M3 scale per 16 contiguous elements, one FP32 tensor scale;
// optional random 16x16 Hadamard transform along the quantized dimension and
// stochastic rounding.
//
// "NVIDIA developed a method to train neural networks at 4-bit", section
// "How it works": the 4-bit NVFP4 format, random 16x16 Hadamard transforms
// of the gradient inputs, stochastic rounding.  The two-level scale:
//   s_t = fl32(amax_t / 2688)          (2688 = 448 * 6; 1 if amax_t = 0,
//                                       NaN if amax_t is not finite)
//   s_b = E4M3_RNE_SAT(fl32(amax_b / fl32(6 * s_t)))   per 16 elements
//   d   = fl32(dec(s_b) * s_t)
//   code = E2M1(sat6(fl32(x / d)))     RNE (ties to the even code) or
//                                       stochastic; d = 0 or NaN -> code 0
// amax_t is taken over the (transformed) tensor being quantized, so a
// row-wise and a column-wise output have their own tensor scale.
//
// Random Hadamard transform of a 16-chunk: z = d (.) x with the signs d_j
// (-1 where bit j of sign_mask is set), four butterfly stages with strides
// 1, 2, 4, 8 ((a, b) -> (a + b, a - b) in FP32), then the exact factor 1/4.
// Stochastic rounding of |y| between neighbours lo < hi: round up iff
// (r >> 10) < floor(p * 2^22) with p = (|y| - lo) / (hi - lo) (the 22 high
// bits of r against p resolved to 22 bits), where the random word of
// source element i (row * cols + col of x) is
// r = fmix32(lo32(i) ^ fmix32(lo32(seed) ^ fmix32(hi32(seed) ^ hi32(i)))),
// fmix32 being MurmurHash3's 32-bit finalizer.
//
// Two kernels: a tensor-amax pass (both orientations from one read, one
// partial per workgroup and orientation in the workspace) and the quantize
// pass, which takes the max of the partials.  One workgroup (256 threads, 4 waves) owns a 128 x 128
// tile of x; thread t (wave w, lane l) holds the 8 x 8 sub-block with
// columns 8*(l & 15) .. +7 and rows 8*(4w + (l >> 4)) .. +7.  A row-wise
// 16-chunk spans lanes l, l ^ 1; a column-wise one spans lanes l, l ^ 16.
#include "fgs_device.h"
#include "fgs_internal.h"

namespace fgs {

namespace {

constexpr int TB = 128;
constexpr int TPAD = 16;

__device__ __forceinline__ uint32_t fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

__device__ __forceinline__ float bf16_at(const uint4& v, int j)
{
    const uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

__device__ __forceinline__ float xor1(float v)
{
    // every lane is written (full row and bank masks), so no old value is needed
    return as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), DPP_XOR1, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor16(float v)
{
    return __shfl_xor(v, 16);
}

// Random Hadamard transform of the 16-chunk whose elements 8*hpos .. 8*hpos+7
// this lane holds (the partner lane holds the other 8), without the final
// factor 1/4: z holds d (.) x on entry, negated on the hpos 1 lane (the
// signs are applied to the packed BF16 pairs, see rht_pair_signs), and
// 4 * (H d x) on return.  The caller folds the exact 1/4 into the block amax
// and the divisor.  The three in-lane stages carry the negation through
// exactly (nearest rounding is symmetric), so the stride-8 stage is
// z + s * partner with s = -1 on hpos 0 (giving a + b) and +1 on hpos 1
// (giving a - b), one FMA whose product by +-1 is exact.  Row-wise the
// partner is the neighbouring lane, read through a DPP operand of the FMA.
template <bool ROWWISE>
__device__ __forceinline__ void rht16x4(float z[8], float s)
{
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const float a = z[i], b = z[i + h];
                z[i] = a + b;
                z[i + h] = a - b;
            }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float other = ROWWISE ? xor1(z[i]) : xor16(z[i]);
        z[i] = __builtin_fmaf(other, s, z[i]);
    }
}

// XOR masks that apply the RHT signs to packed BF16 pairs, and negate every
// element on the hpos 1 lane (see rht16x4).  Row-wise chunks run along the
// 8 columns of a lane (positions 8*hpos + j, pair k = columns 2k, 2k+1);
// column-wise chunks run along its 8 rows (position 8*hpos + u, the same
// sign for every column of row u).
__device__ __forceinline__ void rht_pair_signs(uint32_t sign_mask, int hpos_row, int hpos_col,
                                               uint32_t row_m[4], uint32_t col_m[8])
{
    const uint32_t sr = sign_mask >> (8 * hpos_row), sc = sign_mask >> (8 * hpos_col);
    const uint32_t nrow = hpos_row ? 0x80008000u : 0u, ncol = hpos_col ? 0x80008000u : 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        row_m[k] = ((((sr >> (2 * k)) & 1u) << 15) | (((sr >> (2 * k + 1)) & 1u) << 31)) ^ nrow;
#pragma unroll
    for (int u = 0; u < 8; ++u) col_m[u] = (((sc >> u) & 1u) * 0x80008000u) ^ ncol;
}

__device__ __forceinline__ uint4 xor4(const uint4& v, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return make_uint4(v.x ^ a, v.y ^ b, v.z ^ c, v.w ^ d);
}

// FP32 bits of a quarter of the FP32 value with bits m (exact for every
// value a transformed chunk can hold; NaN stays NaN, Inf stays Inf)
__device__ __forceinline__ uint32_t quarter_bits(uint32_t m)
{
    return as_u32(as_f32(m) * 0.25f);
}

__device__ __forceinline__ uint32_t fabs_bits(float v) { return as_u32(v) & 0x7FFFFFFFu; }

// max of |z| as FP32 bits (integer order = value order; NaN above Inf)
__device__ __forceinline__ uint32_t amax8(const float z[8])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, fabs_bits(z[i]));
    return m;
}

__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
    return v[0];
}

// Stochastic E2M1 codes of 8 values (element 2k in the low nibble of byte
// k, 2k + 1 in the high nibble) from v_cvt_scalef32_sr_pk_fp4_f32 at unit
// scale.  The instruction converts a pair (lo slot, hi slot) into one byte;
// the lo slot rounds up iff (s >> 10) + floor(p * 2^22) >= 2^22 for its
// random operand s, the hi slot the same with rotl(s, 1), and both keep the
// sign (so -0 gives code 8) and saturate at 6.  With s = ~r the lo slot
// rounds up iff (r >> 10) < floor(p * 2^22), the rule above; the hi slot
// gets it with s = rotr(~r, 1).  Each pair is therefore converted twice,
// once with the even element's operand and once with the odd one's, and
// the nibbles are merged with a bitfield insert: every element rounds with
// its own word.  Checked on gfx950 against the rule in integer arithmetic
// for every FP32 magnitude in [0, 6], both signs, with words at and beside
// each decision boundary, in every one of the 8 positions.  Written as
// inline assembly because the compiler builtin does not tie its old-value
// operand to the destination, which the byte select relies on to keep the
// other three bytes.  nr holds ~r for the 8 values.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int SEL>
__device__ __forceinline__ void cvt_sr_fp4_byte(uint32_t& w, f32x2 v, uint32_t s)
{
    if constexpr (SEL == 0)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(w) : "v"(v), "v"(s));
    else if constexpr (SEL == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(w) : "v"(v), "v"(s));
    else if constexpr (SEL == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(w) : "v"(v), "v"(s));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(w) : "v"(v), "v"(s));
}

__device__ __forceinline__ uint32_t e2m1_sr_pack8(const float v[8], const uint32_t nr[8])
{
    uint32_t ev, od;       // every byte is written by the four calls below
    asm("" : "=v"(ev));
    asm("" : "=v"(od));
    cvt_sr_fp4_byte<0>(ev, f32x2{v[0], v[1]}, nr[0]);
    cvt_sr_fp4_byte<0>(od, f32x2{v[0], v[1]}, __builtin_amdgcn_alignbit(nr[1], nr[1], 1));
    cvt_sr_fp4_byte<1>(ev, f32x2{v[2], v[3]}, nr[2]);
    cvt_sr_fp4_byte<1>(od, f32x2{v[2], v[3]}, __builtin_amdgcn_alignbit(nr[3], nr[3], 1));
    cvt_sr_fp4_byte<2>(ev, f32x2{v[4], v[5]}, nr[4]);
    cvt_sr_fp4_byte<2>(od, f32x2{v[4], v[5]}, __builtin_amdgcn_alignbit(nr[5], nr[5], 1));
    cvt_sr_fp4_byte<3>(ev, f32x2{v[6], v[7]}, nr[6]);
    cvt_sr_fp4_byte<3>(od, f32x2{v[6], v[7]}, __builtin_amdgcn_alignbit(nr[7], nr[7], 1));
    return (ev & 0x0F0F0F0Fu) | (od & 0xF0F0F0F0u);
}

// E2M1 codes of 8 quotients, packed: stochastic from e2m1_sr_pack8, or RNE
// from v_cvt_scalef32_pk_fp4_f32 (unit scale), which for every FP32 value in
// [-6, 6] gives the nearest magnitude of {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties
// to the even code) with the sign of the input, and saturates at 6 beyond
// (both checked exhaustively on gfx950).
template <bool SR>
__device__ __forceinline__ uint32_t e2m1_pack8(const float v[8], const uint32_t nr[8])
{
    if constexpr (SR) {
        return e2m1_sr_pack8(v, nr);
    } else {
        uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
        return w;
    }
}

struct TensorScale {
    float st, six_st, r6;    // s_t, fl32(6 s_t), RN(1 / fl32(6 s_t))
};

__device__ __forceinline__ TensorScale tensor_scale_from(uint32_t amax_bits)
{
    TensorScale s;
    if (amax_bits >= 0x7F800000u) s.st = __builtin_nanf("");
    else if (amax_bits == 0) s.st = 1.0f;
    else s.st = as_f32(amax_bits) / 2688.0f;
    s.six_st = 6.0f * s.st;
    s.r6 = 1.0f / s.six_st;
    return s;
}

// fl32(a / d) for a >= 0 from r = RN(1/d): Markstein's correction
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Dev., 1990): q0 = RN(a r), the
// residual a - q0 d is exact with an FMA, and RN(q0 + residual * r) is the
// correctly rounded quotient while the residual stays a normal number.
// Checked against IEEE division on gfx950 for every BF16 a >= 2^-90 with
// every divisor mantissa of three binades and for 1.7e10 random FP32 pairs.
__device__ __forceinline__ float div_rn(float a, float d, float r)
{
    const float q0 = a * r;
    const float res = __builtin_fmaf(-q0, d, a);
    return __builtin_fmaf(res, r, q0);
}

// Codes of 8 values of one 16-block whose (two-lane) amax bits are amax_b.
// Returns the 8 nibbles packed (element 2j in the low nibble) and the scale
// byte.  Waves whose blocks are all ordinary take the fast path below; on
// the careful path the quotient y / d is taken on |y| with the sign put back
// bitwise (so -0 gives the negative-zero code 0x8) and saturated at 6.  A block with
// amax_b < 2^-30 divides y * 2^64 by d * 2^64 (both exact), which keeps every
// residual normal; in other blocks an element below 2^-90 has a quotient
// below 2^-57, where RNE gives 0 and stochastic rounding never rounds up
// (floor(p * 2^22) = 0), so its rounding cannot change a code.  RNE codes
// come from e2m1_pack8 (the hardware converters), with nr the complements
// ~r of the elements' words for stochastic rounding.
//
// y = z / zscale: z is either the value itself (zscale 1) or four times the
// transformed value (zscale 4, see rht16x4); amax_b is the amax of y.  The
// quotient fl32(y / d) is the correctly rounded z / (zscale d), and zscale d
// is exact (d <= 448 * 2^128 / 2688 leaves room for the factor 4).
template <bool SR>
__device__ __forceinline__ uint32_t nv_block8(const float y[8], uint32_t amax_b, const TensorScale& ts,
                                              const uint32_t nr[8], uint32_t& sb_out, float zscale)
{
    // fl32(amax_b / (6 s_t)) by the same correction as the elements (the
    // residual is normal for amax_b >= 2^-90; smaller block maxima take IEEE
    // division), then the hardware E4M3 cast: the quotient is at most
    // 448 (1 + 2^-23) because amax_b <= amax_t, and the min with 448 makes
    // the cast saturate exactly as the encoder does.
    const float amb = as_f32(amax_b);
    // Wave-uniform fast path: every lane's block has a finite amax of at
    // least 2^-30 and a nonzero, finite d.  Then the scale quotient takes
    // the correction, no element needs the 2^64 pre-scale, the quotients
    // are taken on the signed values (div_by_scale: sign-symmetric and
    // equal to div_rn on |y|, -0 kept) and the converters saturate beyond 6
    // by themselves (checked on gfx950 for every FP32 magnitude above 6).
    {
        const float qs = div_rn(amb, ts.six_st, ts.r6);
        const uint32_t sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(qs, 448.0f), 0.0f, 0, false) & 0xFFu;
        const float d = e4m3_value(sb) * ts.st;
        const bool ok = amax_b >= 0x30800000u && amax_b < 0x7F800000u && d > 0.0f;
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
            sb_out = sb;
            const float dk = d * zscale;
            const float r = 1.0f / dk;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = div_by_scale(y[i], dk, r);
            return e2m1_pack8<SR>(v, nr);
        }
    }
    float qs;
    if (__builtin_expect(amb >= 0x1p-90f, 1)) qs = div_rn(amb, ts.six_st, ts.r6);
    else qs = amb / ts.six_st;
    uint32_t sb;
    if (qs != qs) sb = 0x7Fu;
    else sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(qs, 448.0f), 0.0f, 0, false) & 0xFFu;
    sb_out = sb;
    const float d = e4m3_value(sb) * ts.st;
    if (d == 0.0f || d != d) return 0;
    float k = 1.0f;
    if (__builtin_expect(as_f32(amax_b) < 0x1p-30f, 0)) k = 0x1p64f;
    const float dk = d * zscale * k;
    const float r = 1.0f / dk;
    float q[8];
    uint32_t sg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a = __builtin_fabsf(y[i]);
        if (__builtin_expect(k != 1.0f, 0)) a *= k;
        q[i] = __builtin_fminf(div_rn(a, dk, r), 6.0f);
        sg[i] = as_u32(y[i]) & 0x80000000u;
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = as_f32(as_u32(q[i]) | sg[i]);
    return e2m1_pack8<SR>(v, nr);
}

// The counter hash's last round: r = fmix32(lo32(i) ^ mid) with
// mid = fmix32(lo32(seed) ^ fmix32(hi32(seed) ^ hi32(i))), which is the same
// for every element whose index has the same upper 32 bits.
__device__ __forceinline__ uint32_t sr_mid(uint32_t seed_lo, uint32_t seed_hi, uint64_t i)
{
    return fmix32(seed_lo ^ fmix32(seed_hi ^ (uint32_t)(i >> 32)));
}

// Random word of element i0 + j (0 <= j < 8) from base = lo32(i0) ^ mid0,
// mid0 the seed rounds of i0.  Every run of 8 starts at a multiple of 8
// (cols and the column offset are multiples of 8), so lo32(i0) + j equals
// lo32(i0) ^ j, never carries into hi32, and the seed rounds of i0 hold for
// the whole run: fmix32((lo32(i0) + j) ^ mid0) = fmix32(base ^ j).
__device__ __forceinline__ uint32_t sr_word_at(uint32_t base, int j)
{
    return fmix32(base ^ (uint32_t)j);
}

__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                          int64_t r0, int64_t col, int rg, bool col_ok, uint4 v[8])
{
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t row = r0 + 8 * rg + u;
        if (col_ok && row < rows)
            v[u] = load_nt16(x + row * ldx + col);
        else
            v[u] = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------- pass 1 --
// max |x| of 8 BF16 values as FP32 bits (BF16 magnitude order is FP32 order;
// NaN above Inf)
__device__ __forceinline__ uint32_t bf16_amax8_bits(const uint4& v)
{
    const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
    const uint32_t m = max(max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16)),
                           max(max(c & 0xFFFFu, c >> 16), max(d & 0xFFFFu, d >> 16)));
    return m << 16;
}

// Tensor amax of both orientations (of the transformed values where the
// transform applies).  Persistent over 128 x 128 tiles with stride
// gridDim.x, the next tile's rows loaded before the current one is reduced;
// each workgroup stores its two maxima to ws[2 * blockIdx.x + o] (o = 0
// row-wise, 1 column-wise): no same-address atomics, no clearing pass.
__global__ __launch_bounds__(256) void nvfp4_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    int rht_mask, uint32_t sign_mask, uint32_t* __restrict__ ws)
{
    __shared__ uint32_t red[2][4];
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = l & 15, rg = 4 * w + (l >> 4);
    const int64_t nbc = (cols + TB - 1) / TB, nblk = ((rows + TB - 1) / TB) * nbc;
    uint32_t row_m[4], col_m[8];
    rht_pair_signs(sign_mask, cg & 1, (l >> 4) & 1, row_m, col_m);
    const float sgn_row = (cg & 1) ? 1.0f : -1.0f, sgn_col = ((l >> 4) & 1) ? 1.0f : -1.0f;
    const bool rht_row = rht_mask & 1, rht_col = rht_mask & 2;

    uint32_t plain = 0, mrow4 = 0, mcol4 = 0;     // mrow4 / mcol4: amax of 4 x the transform
    int64_t blk = blockIdx.x;
    uint4 v[8];
    if (blk < nblk) {
        const int64_t col = (blk % nbc) * TB + 8 * cg;
        load_tile(x, rows, cols, ldx, (blk / nbc) * TB, col, rg, col < cols, v);
    }
    while (blk < nblk) {
        const int64_t next = blk + gridDim.x;
        uint4 vn[8];
        if (next < nblk) {
            const int64_t col = (next % nbc) * TB + 8 * cg;
            load_tile(x, rows, cols, ldx, (next / nbc) * TB, col, rg, col < cols, vn);
        }
        if (!(rht_row && rht_col)) {
#pragma unroll
            for (int u = 0; u < 8; ++u) plain = max(plain, bf16_amax8_bits(v[u]));
        }
        if (rht_row) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint4 vs = xor4(v[u], row_m[0], row_m[1], row_m[2], row_m[3]);
                float z[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) z[jj] = bf16_at(vs, jj);
                rht16x4<true>(z, sgn_row);
                mrow4 = max(mrow4, amax8(z));
            }
        }
        if (rht_col) {
            uint4 vs[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) vs[u] = xor4(v[u], col_m[u], col_m[u], col_m[u], col_m[u]);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                float z[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) z[u] = bf16_at(vs[u], jj);
                rht16x4<false>(z, sgn_col);
                mcol4 = max(mcol4, amax8(z));
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = vn[u];
        blk = next;
    }
    uint32_t mrow = rht_row ? quarter_bits(mrow4) : plain;
    uint32_t mcol = rht_col ? quarter_bits(mcol4) : plain;
    mrow = max_xor32(max_xor16(max_lanes16(mrow)));
    mcol = max_xor32(max_xor16(max_lanes16(mcol)));
    if (l == 0) {
        red[0][w] = mrow;
        red[1][w] = mcol;
    }
    __syncthreads();
    if (t < 2) ws[2 * blockIdx.x + t] = max(max(red[t][0], red[t][1]), max(red[t][2], red[t][3]));
}

// ---------------------------------------------------------------- pass 2 --
template <bool SR>
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    int rht_mask, uint32_t sign_mask, uint32_t seed_lo, uint32_t seed_hi,
    uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ qT, uint8_t* __restrict__ scalesT,
    float* __restrict__ tensor_scale, const uint32_t* __restrict__ ws, int32_t n_amax)
{
    __shared__ __align__(16) uint8_t tbuf[TB][TB / 2 + TPAD];
    __shared__ uint32_t s_red[2][4];
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = l & 15, rg = 4 * w + (l >> 4);
    const int64_t r0 = (int64_t)blockIdx.y * TB, c0 = (int64_t)blockIdx.x * TB;
    const int64_t col = c0 + 8 * cg;
    const bool col_ok = col < cols;
    uint4 v[8];
    load_tile(x, rows, cols, ldx, r0, col, rg, col_ok, v);

    // tensor amax of each orientation: the max of the amax pass's partials
    // (read after this tile's loads are in flight)
    uint32_t mr = 0, mc = 0;
    for (int i = t; i < n_amax; i += 256) {
        mr = max(mr, ws[2 * i]);
        mc = max(mc, ws[2 * i + 1]);
    }
    mr = max_xor32(max_xor16(max_lanes16(mr)));
    mc = max_xor32(max_xor16(max_lanes16(mc)));
    if (l == 0) {
        s_red[0][w] = mr;
        s_red[1][w] = mc;
    }
    __syncthreads();
    const TensorScale ts_row = tensor_scale_from(max(max(s_red[0][0], s_red[0][1]), max(s_red[0][2], s_red[0][3])));
    const TensorScale ts_col = tensor_scale_from(max(max(s_red[1][0], s_red[1][1]), max(s_red[1][2], s_red[1][3])));
    // SR: the random word of an element does not depend on the
    // orientation: hash each of the thread's 64 elements once for both
    // outputs (the seed rounds once per row of the thread), kept as ~r, the
    // converter's operand
    uint32_t W[8][8];
    if constexpr (SR) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint64_t i0 = (uint64_t)((r0 + 8 * rg + u) * cols + col);
            const uint32_t base = (uint32_t)i0 ^ sr_mid(seed_lo, seed_hi, i0);
#pragma unroll
            for (int j = 0; j < 8; ++j) W[u][j] = ~sr_word_at(base, j);
        }
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) {
        tensor_scale[0] = ts_row.st;
        tensor_scale[1] = ts_col.st;
    }

    uint32_t row_m[4], col_m[8];
    rht_pair_signs(sign_mask, cg & 1, (l >> 4) & 1, row_m, col_m);

    // ---------------- row-wise: 16-blocks along columns ----------------
    if (q) {
        const int64_t qcols = cols / 2, nsc = cols / 16;
        const bool rht = rht_mask & 1;
        const float sgn = (cg & 1) ? 1.0f : -1.0f, zscale = rht ? 4.0f : 1.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float z[8];
            const uint4 vs = rht ? xor4(v[u], row_m[0], row_m[1], row_m[2], row_m[3]) : v[u];
#pragma unroll
            for (int j = 0; j < 8; ++j) z[j] = bf16_at(vs, j);
            if (rht) rht16x4<true>(z, sgn);
            uint32_t mb = amax8(z);
            const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, DPP_XOR1, 0xF, 0xF, false);
            mb = max(mb, other);
            if (rht) mb = quarter_bits(mb);
            const int64_t row = r0 + 8 * rg + u;
            uint32_t rw[8];
            if constexpr (SR) {
#pragma unroll
                for (int j = 0; j < 8; ++j) rw[j] = W[u][j];
            }
            uint32_t sb;
            const uint32_t packed = nv_block8<SR>(z, mb, ts_row, rw, sb, zscale);
            if (col_ok && row < rows) {
                *reinterpret_cast<uint32_t*>(q + row * qcols + col / 2) = packed;
                if (!(cg & 1)) scales[row * nsc + col / 16] = (uint8_t)sb;
            }
        }
    }

    // ---------------- column-wise: 16-blocks along rows ----------------
    if (qT) {
        const int64_t nscT = rows / 16;
        const int hpos = (l >> 4) & 1;
        const bool rht = rht_mask & 2;
        const float sgn = hpos ? 1.0f : -1.0f, zscale = rht ? 4.0f : 1.0f;
        if (rht) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = xor4(v[u], col_m[u], col_m[u], col_m[u], col_m[u]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float z[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) z[u] = bf16_at(v[u], j);
            if (rht) rht16x4<false>(z, sgn);
            uint32_t mb = amax8(z);
            mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
            if (rht) mb = quarter_bits(mb);
            uint32_t rw[8];
            if constexpr (SR) {
#pragma unroll
                for (int u = 0; u < 8; ++u) rw[u] = W[u][j];
            }
            uint32_t sb;
            const uint32_t packed = nv_block8<SR>(z, mb, ts_col, rw, sb, zscale);
            *reinterpret_cast<uint32_t*>(&tbuf[8 * cg + j][4 * rg]) = packed;
            if (hpos == 0 && col_ok) scalesT[(col + j) * nscT + (r0 + 8 * rg) / 16] = (uint8_t)sb;
        }
        __syncthreads();
        // 4 lanes write one 64-byte row of qT
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int trow = 64 * i + (t >> 2), chunk = t & 3;
            const int64_t orow = c0 + trow;
            if (orow < cols) {
                const uint4 d = *reinterpret_cast<const uint4*>(&tbuf[trow][16 * chunk]);
                *reinterpret_cast<uint4*>(qT + orow * (rows / 2) + r0 / 2 + 16 * chunk) = d;
            }
        }
    }
}

// Sign mask of the random Hadamard transform: bit j set <=> d_j = -1, with
// d_j from bit 0 of fmix32(j ^ key), key = fmix32(lo32(seed) ^ fmix32(hi32(seed))).
uint32_t host_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

uint32_t rht_sign_mask(uint64_t seed)
{
    const uint32_t key = host_fmix32((uint32_t)seed ^ host_fmix32((uint32_t)(seed >> 32)));
    uint32_t m = 0;
    for (uint32_t j = 0; j < 16; ++j) m |= (host_fmix32(j ^ key) & 1u) << j;
    return m;
}

} // namespace

hipError_t launch_quant_nvfp4(const QuantNVFP4Args& a, hipStream_t stream)
{
    const int64_t nbr = (a.rows + TB - 1) / TB, nbc = (a.cols + TB - 1) / TB;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const dim3 grid((unsigned)nbc, (unsigned)nbr), block(256);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    uint32_t* ws = static_cast<uint32_t*>(a.workspace);
    const uint32_t mask = rht_sign_mask(a.rht_seed);
    // amax workgroups: two per compute unit, at most one per 8-byte
    // workspace slot (two partials each)
    int64_t g = nbr * nbc;
    const int64_t cap = (int64_t)device_cus() * 2, slots = (int64_t)(a.workspace_bytes / 8);
    if (g > cap) g = cap;
    if (g > slots) g = slots;
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)g), block, 0, stream,
                       x, a.rows, a.cols, a.ldx, a.rht_mask, mask, ws);
    const uint32_t slo = (uint32_t)a.sr_seed, shi = (uint32_t)(a.sr_seed >> 32);
    if (a.stochastic)
        hipLaunchKernelGGL(nvfp4_quant_kernel<true>, grid, block, 0, stream, x, a.rows, a.cols, a.ldx, a.rht_mask,
                           mask, slo, shi, a.q, a.scales, a.qT, a.scalesT, a.tensor_scale, ws, (int32_t)g);
    else
        hipLaunchKernelGGL(nvfp4_quant_kernel<false>, grid, block, 0, stream, x, a.rows, a.cols, a.ldx, a.rht_mask,
                           mask, slo, shi, a.q, a.scales, a.qT, a.scalesT, a.tensor_scale, ws, (int32_t)g);
    return hipGetLastError();
}

} // namespace fgs
