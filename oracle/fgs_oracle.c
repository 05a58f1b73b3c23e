/*
 * fgs_oracle.c -- plain CPU oracle for fine-grained scaled low-precision
 * quantization (E4M3 tiles/blocks/tensor, MXFP8, NVFP4 with the random
 * Hadamard transform and stochastic rounding).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or table with the GPU library; it is written to be read against
 * the source pages, not to be fast.
 *
 * Sources (cited by page title and section):
 *  [DSV3]  "Can you explain the role of FP8 precision in DeepSeek-V3
 *          training" (codingmall.com knowledge base), sections
 *          "Fine-grained quantization", "Online quantization",
 *          "Increasing accumulation precision", "Unified E4M3 format".
 *  [NEMO]  "Accelerating FP8 training performance with the NVIDIA NeMo
 *          framework" (hyper.ai headline), body: recipes, MXFP8 blocks of 32,
 *          per-tensor vs block-wise scaling.
 *  [NVFP4] "NVIDIA developed a method to train neural networks at 4-bit"
 *          (news.hamidun.com), section "How it works": NVFP4, random 16x16
 *          Hadamard transforms of gradient inputs, stochastic rounding.
 *  The pages name the formats but do not define their bits; the element
 *  codecs follow the public OCP 8-bit floating point (E4M3FN) and OCP
 *  microscaling (E2M1, E8M0) definitions.  Every point the pages leave open
 *  is read the plainest way; each reading is marked READING below.
 *
 * Precision: scale and quotient arithmetic is IEEE binary32 with
 * round-to-nearest-even, as fixed by the method's scale rule
 * (scale = amax/448 computed in FP32); everything else is exact.  Build
 * with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* BF16 (upper half of an IEEE binary32)                               */
/* ------------------------------------------------------------------ */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------ */
/* E4M3 (OCP E4M3FN): s.eeee.mmm, bias 7, no infinities,               */
/* S.1111.111 is NaN.  [DSV3 "Unified E4M3 format"] names the format.  */
/* ------------------------------------------------------------------ */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);            /* subnormal: m * 2^-9       */
    else
        v = ldexp(8.0 + m, e - 10);          /* (1 + m/8) * 2^(e-7)       */
    return s ? -v : v;
}

/*
 * Round an FP32 value to E4M3: nearest representable value, ties to the
 * even code, saturating at +-448 (the largest finite code 0x7E).
 * READING: overflow saturates instead of producing NaN (the method casts
 * "with saturation"); NaN maps to 0x7F; the sign is kept, so -0 -> 0x80.
 */
uint8_t orc_e4m3_encode(float y)
{
    uint8_t sign;
    double a, lo, hi, mid;
    int c, lo_i, hi_i;

    if (isnan(y))
        return 0x7F;
    sign = signbit(y) ? 0x80 : 0x00;
    a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7E;
    /* Non-negative finite codes 0x00..0x7E are in ascending value order:
     * find the largest code whose value is <= a by bisection. */
    lo_i = 0;
    hi_i = 0x7E;
    while (lo_i < hi_i) {
        c = (lo_i + hi_i + 1) / 2;
        if (orc_e4m3_decode((uint8_t)c) <= a)
            lo_i = c;
        else
            hi_i = c - 1;
    }
    c = lo_i;
    lo = orc_e4m3_decode((uint8_t)c);
    if (a == lo)
        return sign | (uint8_t)c;
    hi = orc_e4m3_decode((uint8_t)(c + 1));
    mid = 0.5 * (lo + hi);                   /* exact: both have <= 4 bits */
    if (a < mid)
        return sign | (uint8_t)c;
    if (a > mid)
        return sign | (uint8_t)(c + 1);
    return sign | (uint8_t)((c & 1) ? c + 1 : c);   /* tie: even code */
}

/* ------------------------------------------------------------------ */
/* E5M2 (OCP FP8): s.eeeee.mm, bias 15, subnormals, 0x7C = Inf,          */
/* 0x7D..0x7F NaN, largest finite 0x7B = 57344.  The pages contrast       */
/* DeepSeek-V3's single E4M3 format with earlier hybrid recipes (E4M3     */
/* forward, E5M2 backward) [DSV3 "Unified E4M3 format"].                  */
/* ------------------------------------------------------------------ */
double orc_e5m2_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 0x1F, m = c & 0x3;
    double v;
    if (e == 0x1F)
        return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0)
        v = ldexp((double)m, -16);           /* subnormal: m * 2^-16      */
    else
        v = ldexp(4.0 + m, e - 17);          /* (1 + m/4) * 2^(e-15)      */
    return s ? -v : v;
}

/*
 * Round an FP32 value to E5M2: nearest representable value, ties to the
 * even code, saturating at +-57344.
 * READING: as for E4M3, the cast saturates (overflow and +-Inf give
 * +-57344, never Inf); NaN maps to 0x7F; the sign is kept (-0 -> 0x80).
 */
uint8_t orc_e5m2_encode(float y)
{
    uint8_t sign;
    double a, lo, hi, mid;
    int c, lo_i, hi_i;

    if (isnan(y))
        return 0x7F;
    sign = signbit(y) ? 0x80 : 0x00;
    a = fabs((double)y);
    if (a >= 57344.0)
        return sign | 0x7B;
    lo_i = 0;
    hi_i = 0x7B;
    while (lo_i < hi_i) {                    /* largest code with value <= a */
        c = (lo_i + hi_i + 1) / 2;
        if (orc_e5m2_decode((uint8_t)c) <= a)
            lo_i = c;
        else
            hi_i = c - 1;
    }
    c = lo_i;
    lo = orc_e5m2_decode((uint8_t)c);
    if (a == lo)
        return sign | (uint8_t)c;
    hi = orc_e5m2_decode((uint8_t)(c + 1));
    mid = 0.5 * (lo + hi);
    if (a < mid)
        return sign | (uint8_t)c;
    if (a > mid)
        return sign | (uint8_t)(c + 1);
    return sign | (uint8_t)((c & 1) ? c + 1 : c);
}

/* ------------------------------------------------------------------ */
/* E2M1 (OCP FP4): s.ee.m, magnitudes {0,.5,1,1.5,2,3,4,6}, no NaN/Inf  */
/* [NVFP4 "How it works"] names the 4-bit format.                      */
/* ------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint8_t c)
{
    double v = E2M1_MAG[c & 0x7];
    return (c & 0x8) ? -v : v;
}

/* index of the largest magnitude <= a (a in [0, 6]) */
static int e2m1_floor_index(double a)
{
    int i = 0;
    while (i < 7 && E2M1_MAG[i + 1] <= a)
        i++;
    return i;
}

/* Round to E2M1, nearest, ties to the even code, saturating at +-6.
 * READING: the sign is kept (a negative value that rounds to zero gives
 * code 0x8), matching the E4M3 rule above. */
uint8_t orc_e2m1_encode_rne(float y)
{
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    double a = fabs((double)y), lo, hi, mid;
    int i;
    if (isnan(y))
        return 0x0;
    if (a >= 6.0)
        return sign | 0x7;
    i = e2m1_floor_index(a);
    lo = E2M1_MAG[i];
    if (a == lo)
        return sign | (uint8_t)i;
    hi = E2M1_MAG[i + 1];
    mid = 0.5 * (lo + hi);
    if (a < mid)
        return sign | (uint8_t)i;
    if (a > mid)
        return sign | (uint8_t)(i + 1);
    return sign | (uint8_t)((i & 1) ? i + 1 : i);
}

/*
 * Stochastic rounding to E2M1 with a 32-bit random word r.
 * READING [NVFP4 "How it works" names stochastic rounding only, not its
 * resolution]: with lo <= |y| < hi the two neighbouring magnitudes and
 * p = (|y| - lo) / (hi - lo), round up iff (r >> 10) < floor(p * 2^22).
 * The 22 high bits of r are the uniform variate and p is resolved to 22
 * bits, so P(up) = floor(p * 2^22) / 2^22: exactly p for |y| >= 1, where
 * p * 2^22 is an integer, and less than 2^-22 below p for |y| < 1.  p and
 * floor(p * 2^22) are exact in double.  Values already representable never
 * move; |y| >= 6 saturates.
 */
uint8_t orc_e2m1_encode_sr(float y, uint32_t r)
{
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    double a = fabs((double)y), lo, hi, p;
    int i;
    if (isnan(y))
        return 0x0;
    if (a >= 6.0)
        return sign | 0x7;
    i = e2m1_floor_index(a);
    lo = E2M1_MAG[i];
    if (a == lo)
        return sign | (uint8_t)i;
    hi = E2M1_MAG[i + 1];
    p = (a - lo) / (hi - lo);
    if ((double)(r >> 10) < floor(p * 4194304.0))
        return sign | (uint8_t)(i + 1);
    return sign | (uint8_t)i;
}

/* E8M0: 2^(c-127), c = 255 is NaN.  [NEMO] "blocks of 32 values". */
double orc_e8m0_decode(uint8_t c)
{
    if (c == 0xFF)
        return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* ------------------------------------------------------------------ */
/* Counter-based hash: MurmurHash3's 32-bit finalizer (public domain,   */
/* Austin Appleby).  Used for the SR random words and the RHT signs.   */
/* ------------------------------------------------------------------ */
uint32_t orc_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

/* Random word for element i (linear index in the source tensor). */
uint32_t orc_sr_word(uint64_t seed, uint64_t i)
{
    uint32_t inner = orc_fmix32((uint32_t)(seed >> 32) ^ (uint32_t)(i >> 32));
    uint32_t mid = orc_fmix32((uint32_t)seed ^ inner);
    return orc_fmix32((uint32_t)i ^ mid);
}

/* Sign vector of the random Hadamard transform: d_j = -1 iff bit 0 of
 * fmix32(j ^ key) is set, key = fmix32(lo32(seed) ^ fmix32(hi32(seed))). */
void orc_rht_signs(uint64_t seed, float d[16])
{
    uint32_t key = orc_fmix32((uint32_t)seed ^ orc_fmix32((uint32_t)(seed >> 32)));
    int j;
    for (j = 0; j < 16; j++)
        d[j] = (orc_fmix32((uint32_t)j ^ key) & 1u) ? -1.0f : 1.0f;
}

/*
 * Random 16x16 Hadamard transform of one 16-vector, in FP32:
 * y = (1/4) * H16 * diag(d) * x with H16 the Sylvester Hadamard matrix.
 * [NVFP4 "How it works"]: random 16x16 Hadamard transforms of the gradient
 * inputs.  READING: orthonormal 1/4 factor; the FP32 result is defined by
 * the fast Walsh-Hadamard evaluation order: strides 1, 2, 4, 8, each pair
 * (a, b) -> (a + b, a - b), then the exact multiply by 1/4.
 */
void orc_rht16(const float *x, const float d[16], float *y)
{
    float z[16];
    int i, h;
    for (i = 0; i < 16; i++)
        z[i] = d[i] * x[i];                 /* exact sign flip */
    for (h = 1; h < 16; h *= 2) {
        for (i = 0; i < 16; i++) {
            if (i & h)
                continue;
            {
                float a = z[i], b = z[i + h];
                z[i] = a + b;
                z[i + h] = a - b;
            }
        }
    }
    for (i = 0; i < 16; i++)
        y[i] = 0.25f * z[i];                /* exact power-of-two scale */
}

/* Apply the RHT to each 16-chunk of every row of x [rows x cols]. */
void orc_rht_rows(const float *x, int64_t rows, int64_t cols, uint64_t seed, float *y)
{
    float d[16];
    int64_t r, c;
    orc_rht_signs(seed, d);
    for (r = 0; r < rows; r++)
        for (c = 0; c + 16 <= cols; c += 16)
            orc_rht16(x + r * cols + c, d, y + r * cols + c);
}

/* ------------------------------------------------------------------ */
/* amax: NaN-propagating maximum of |x|                                 */
/* ------------------------------------------------------------------ */
static float amax_update(float m, float v)
{
    float a = fabsf(v);
    if (isnan(m) || isnan(a))
        return NAN;
    return a > m ? a : m;
}

/*
 * FP32-scaled E4M3 quantization over rectangular blocks of br x bc
 * elements of x [rows x cols] (BF16 bits, row-major).  One scale per block.
 *   tile 1x128  : br = 1,    bc = 128     [DSV3 "Fine-grained quantization"]
 *   block 128x128: br = 128, bc = 128     [DSV3 "Fine-grained quantization"]
 *   per tensor  : br = rows, bc = cols    [NEMO body: per-tensor recipe]
 * Online: the scale comes from the block's own amax at quantization time
 * [DSV3 "Online quantization"].
 *   amax non-finite -> scale NaN, every code 0x7F        (READING)
 *   amax == 0       -> scale 1, codes are signed zeros    (READING)
 *   otherwise       -> s = fl32(amax / 448), q = E4M3(fl32(x / s))
 * Partial blocks at the edges use the elements present (READING).
 * q: [rows x cols]; scales: [ceil(rows/br) x ceil(cols/bc)], row-major.
 */
void orc_quant_e4m3_blocks(const uint16_t *x, int64_t rows, int64_t cols,
                           int64_t br, int64_t bc, uint8_t *q, float *scales)
{
    int64_t nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
    int64_t bi, bj, r, c;
    for (bi = 0; bi < nbr; bi++) {
        for (bj = 0; bj < nbc; bj++) {
            int64_t r0 = bi * br, r1 = r0 + br < rows ? r0 + br : rows;
            int64_t c0 = bj * bc, c1 = c0 + bc < cols ? c0 + bc : cols;
            float amax = 0.0f, s;
            for (r = r0; r < r1; r++)
                for (c = c0; c < c1; c++)
                    amax = amax_update(amax, orc_bf16_to_f32(x[r * cols + c]));
            if (!isfinite(amax))
                s = NAN;
            else if (amax == 0.0f)
                s = 1.0f;
            else
                s = amax / 448.0f;
            scales[bi * nbc + bj] = s;
            for (r = r0; r < r1; r++) {
                for (c = c0; c < c1; c++) {
                    float v = orc_bf16_to_f32(x[r * cols + c]);
                    if (!isfinite(amax))
                        q[r * cols + c] = 0x7F;
                    else
                        q[r * cols + c] = orc_e4m3_encode(v / s);
                }
            }
        }
    }
}

/*
 * MXFP8: E4M3 elements with one E8M0 power-of-two scale per 32 contiguous
 * elements along cols [NEMO body: MXFP8, blocks of 32 values].
 * READING: the scale is the smallest power of two 2^e with amax <= 448 * 2^e
 * (the power-of-two counterpart of amax/448), e clamped to [-127, 127];
 * code = e + 127; q = E4M3(fl32(x * 2^-e)).  amax non-finite -> code 0xFF and
 * NaN codes; amax == 0 -> code 127 and signed zeros.
 * q: [rows x cols]; scales: [rows x ceil(cols/32)].
 */
void orc_quant_mx(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q, uint8_t *scales)
{
    int64_t nb = (cols + 31) / 32, r, b, c;
    for (r = 0; r < rows; r++) {
        for (b = 0; b < nb; b++) {
            int64_t c0 = b * 32, c1 = c0 + 32 < cols ? c0 + 32 : cols;
            float amax = 0.0f;
            int e;
            for (c = c0; c < c1; c++)
                amax = amax_update(amax, orc_bf16_to_f32(x[r * cols + c]));
            if (!isfinite(amax)) {
                scales[r * nb + b] = 0xFF;
                for (c = c0; c < c1; c++)
                    q[r * cols + c] = 0x7F;
                continue;
            }
            if (amax == 0.0f) {
                e = 0;
            } else {
                /* smallest integer e with amax <= 448 * 2^e (exact in double) */
                e = -160;
                while (!((double)amax <= ldexp(448.0, e)))
                    e++;
                if (e < -127)
                    e = -127;
                if (e > 127)
                    e = 127;
            }
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (c = c0; c < c1; c++) {
                float v = orc_bf16_to_f32(x[r * cols + c]);
                q[r * cols + c] = orc_e4m3_encode(ldexpf(v, -e));
            }
        }
    }
}

/*
 * NVFP4 tensor scale [NVFP4 "How it works"].
 * READING (two-level scale): s_t = fl32(amax_t / 2688) with 2688 = 448 * 6,
 * so the tensor amax maps to the top of the E4M3-scale x E2M1 range;
 * amax_t == 0 -> s_t = 1; amax_t non-finite -> s_t = NaN.
 * x holds the n FP32 values being quantized (BF16 inputs widened, possibly
 * Hadamard-transformed).
 */
float orc_nvfp4_tensor_scale(const float *x, int64_t n)
{
    float amax_t = 0.0f;
    int64_t i;
    for (i = 0; i < n; i++)
        amax_t = amax_update(amax_t, x[i]);
    if (!isfinite(amax_t))
        return NAN;
    if (amax_t == 0.0f)
        return 1.0f;
    return amax_t / 2688.0f;
}

/*
 * NVFP4 blocks: E2M1 elements, one E4M3 scale per 16 contiguous elements
 * along cols, under the tensor scale s_t [NVFP4 "How it works"].
 * Per block s_b = E4M3(fl32(amax_b / fl32(6 * s_t))), d = fl32(dec(s_b) * s_t),
 * y = fl32(x / d) saturated to +-6, then E2M1 by RNE or stochastic rounding;
 * d == 0 or NaN -> every code of the block is 0.
 * The SR word of element (r, c) uses the linear index
 * i = idx_base + r * idx_rs + c * idx_cs of that element in the source
 * tensor, so it does not depend on layout, tiling or sampling.
 * q: [rows x ceil(cols/2)] packed, element 2j in the low nibble;
 * scales: [rows x ceil(cols/16)] E4M3 codes.
 */
void orc_quant_nvfp4_blocks(const float *x, int64_t rows, int64_t cols, float s_t,
                            int stochastic, uint64_t sr_seed,
                            int64_t idx_base, int64_t idx_rs, int64_t idx_cs,
                            uint8_t *q, uint8_t *scales)
{
    int64_t nb = (cols + 15) / 16, qc = (cols + 1) / 2, r, b, c;
    memset(q, 0, (size_t)(rows * qc));
    for (r = 0; r < rows; r++) {
        for (b = 0; b < nb; b++) {
            int64_t c0 = b * 16, c1 = c0 + 16 < cols ? c0 + 16 : cols;
            float amax_b = 0.0f, six_st, d;
            uint8_t sb;
            for (c = c0; c < c1; c++)
                amax_b = amax_update(amax_b, x[r * cols + c]);
            six_st = 6.0f * s_t;
            sb = orc_e4m3_encode(amax_b / six_st);
            scales[r * nb + b] = sb;
            d = (float)orc_e4m3_decode(sb) * s_t;
            for (c = c0; c < c1; c++) {
                uint8_t code;
                if (d == 0.0f || isnan(d)) {
                    code = 0;
                } else {
                    float y = x[r * cols + c] / d;
                    if (y > 6.0f)
                        y = 6.0f;
                    if (y < -6.0f)
                        y = -6.0f;
                    if (stochastic)
                        code = orc_e2m1_encode_sr(y, orc_sr_word(sr_seed,
                                   (uint64_t)(idx_base + r * idx_rs + c * idx_cs)));
                    else
                        code = orc_e2m1_encode_rne(y);
                }
                if (c & 1)
                    q[r * qc + c / 2] |= (uint8_t)(code << 4);
                else
                    q[r * qc + c / 2] |= code;
            }
        }
    }
}

/* Whole-tensor NVFP4 quantization: the tensor scale from all of x, then the
 * blocks.  *tensor_scale receives s_t. */
void orc_quant_nvfp4(const float *x, int64_t rows, int64_t cols,
                     int stochastic, uint64_t sr_seed, int64_t idx_rs, int64_t idx_cs,
                     uint8_t *q, uint8_t *scales, float *tensor_scale)
{
    float s_t = orc_nvfp4_tensor_scale(x, rows * cols);
    *tensor_scale = s_t;
    orc_quant_nvfp4_blocks(x, rows, cols, s_t, stochastic, sr_seed, 0, idx_rs, idx_cs, q, scales);
}

/*
 * Per-tensor delayed scaling: the scale comes from the amaxes of earlier
 * steps, not from the tensor being cast.  The pages name it as what online
 * scaling replaces ("delayed quantization methods that depend on
 * historical maximum values") [DSV3 "Online quantization"]; they give no
 * formula.  READING (the plainest one):
 *   hmax = NaN-propagating max of the history (H entries);
 *   hmax non-finite -> scale NaN, every code NaN (0x7F);
 *   hmax == 0 (an empty history) -> scale 1;
 *   otherwise s = fl32(hmax / fmax), fmax = 448 (E4M3) or 57344 (E5M2);
 *   code = ENC_RNE_SAT(fl32(x / s)): values beyond the range of this step's
 *   scale saturate, NaN -> 0x7F;
 *   *amax_out = the NaN-propagating max |x| of this tensor, the entry the
 *   caller records for later steps.
 * x: n BF16 values; q: n codes in the same order.
 */
void orc_quant_delayed(const uint16_t *x, int64_t n, int e5m2, const float *hist, int64_t H,
                       uint8_t *q, float *scale, float *amax_out)
{
    const float fmax = e5m2 ? 57344.0f : 448.0f;
    float hmax = 0.0f, amax = 0.0f, s;
    int64_t i;
    for (i = 0; i < H; i++)
        hmax = amax_update(hmax, hist[i]);
    if (!isfinite(hmax))
        s = NAN;
    else if (hmax == 0.0f)
        s = 1.0f;
    else
        s = hmax / fmax;
    *scale = s;
    for (i = 0; i < n; i++) {
        float v = orc_bf16_to_f32(x[i]);
        amax = amax_update(amax, v);
        if (isnan(s))
            q[i] = 0x7F;
        else
            q[i] = e5m2 ? orc_e5m2_encode(v / s) : orc_e4m3_encode(v / s);
    }
    *amax_out = amax;
}

void orc_e5m2_encode_array(const float *y, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = orc_e5m2_encode(y[i]);
}

/*
 * FP64 -> BF16 with one rounding (RNE): BF16 keeps 8 significant bits and
 * FP32's exponent range (subnormal step 2^-133); overflow past the largest
 * finite value by half an ulp or more gives Inf.  Used for the SwiGLU
 * activation, whose exact value is rounded to the BF16 the next GEMM's
 * quantizer reads.
 */
uint16_t orc_f64_to_bf16(double v)
{
    uint16_t sign;
    double a, q, r;
    int e;
    float f;
    uint32_t b;

    if (isnan(v))
        return 0x7FC0;
    sign = signbit(v) ? 0x8000 : 0x0000;
    a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    frexp(a, &e);                  /* a in [2^(e-1), 2^e) */
    e -= 1;
    if (e < -126)
        e = -126;                  /* subnormal grid */
    q = ldexp(1.0, e - 7);         /* spacing of BF16 numbers at a */
    r = rint(a / q) * q;           /* a / q is exact; rint rounds half to even */
    if (r >= 0x1p128)
        return sign | 0x7F80;
    f = (float)r;                  /* exact: r has <= 8 significant bits */
    memcpy(&b, &f, sizeof b);
    return sign | (uint16_t)(b >> 16);
}

void orc_f64_to_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = orc_f64_to_bf16(v[i]);
}

/* ------------------------------------------------------------------ */
/* Array helpers for the tests (element-wise loops over the codecs).    */
/* ------------------------------------------------------------------ */
void orc_e4m3_encode_array(const float *y, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = orc_e4m3_encode(y[i]);
}

void orc_e2m1_encode_array(const float *y, int64_t n, int stochastic,
                           const uint32_t *r, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = stochastic ? orc_e2m1_encode_sr(y[i], r[i]) : orc_e2m1_encode_rne(y[i]);
}

void orc_sr_word_array(uint64_t seed, const uint64_t *idx, int64_t n, uint32_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = orc_sr_word(seed, idx[i]);
}
