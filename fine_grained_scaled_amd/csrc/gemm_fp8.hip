// gemm_fp8.hip -- block-scaled FP8 (E4M3) GEMM and its grouped (MoE)
// variant on gfx950.
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
// of the two scales is applied once at the end.
//
// Which matrix instruction: gfx950's FP8 MFMA (v_mfma_*_f8f6f4 and the older
// *_fp8_fp8 forms) adds each group of 8 consecutive products with only about
// 13 bits below the largest of them (measured: 256 + 2^-5 survives, 256 +
// 2^-6 does not, and +x - x + tiny gives 0), the same limitation the DeepSeek
// page describes for its hardware, but *inside* one instruction, where no
// promotion interval can reach it.  Its error reaches ~1.5e-4 of
// sum_k |a_k b_k|.  The FP16 MFMA (v_mfma_f32_32x32x16_f16) keeps a full
// FP32-width sum (256 + 2^-15 survives).  Every E4M3 value is exactly an
// FP16 value and every product of two is exact in FP32, so the kernel
// decodes the E4M3 codes to FP16 with the hardware converter
// (v_cvt_scalef32_pk_f16_fp8, unit scale: exact for all 256 codes) and runs
// the FP16 MFMA: the result is the FP32 sum of exact products, promoted per
// 128-K block.
//
// C[m][n] = sum_k A[m][k] * B[n][k]; both operands K-contiguous.
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid, 128 x 128 output tile,
// each wave 64 x 64 = 2 x 2 MFMA 32x32x16 sub-tiles.  K advances in 128-deep
// blocks staged in LDS as FP8 bytes (double-buffered, rows padded to 144
// bytes so the 16-byte fragment reads are bank-conflict free).  MFMA
// operands are swapped (B fragment first) so each lane's 16 accumulators
// share one row m: the 1x128 A scale is then one value per lane.
#include "fgs_device.h"
#include "fgs_internal.h"

namespace fgs {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 16;
constexpr int TILE_BYTES = 128 * LDS_STRIDE;

struct GemmParams {
    const uint8_t* A;
    const uint8_t* B;
    const float* sA;
    const float* sB;
    int64_t lda, ldb, M, N, K;
    int64_t lds_a;        // TILE scales of A: stride between K blocks (= rows of A)
    int64_t lds_b;        // TILE scales of B: stride between K blocks (= rows of B)
    void* C;
    int64_t ldc;
    const int32_t* offsets;
    int32_t G;
    int64_t b_group_stride;       // elements between groups of B codes
    int64_t sb_group_stride;      // floats between groups of B block scales
    int32_t tiles_m, tiles_n;
};

// FP16 x FP16 MFMA, 32x32 outputs, 16-deep K, FP32 accumulate.
__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16 E4M3 codes (one 16-byte LDS read) -> two exact FP16 8-vectors: bytes
// 0..7 feed one MFMA k-step, bytes 8..15 the next.
__device__ __forceinline__ void decode16(const uint8_t* p, f16x8& lo, f16x8& hi)
{
    const uint4 v = *reinterpret_cast<const uint4*>(p);
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

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = as_u32(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;   // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int AMODE, int BMODE, bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(GemmParams p)
{
    __shared__ __align__(16) uint8_t lds[2][2][TILE_BYTES];   // [stage][A|B]
    __shared__ int s_scan[256];
    __shared__ int s_sel[2];

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int wm = w >> 1, wn = w & 1;

    // ------------------------------------------------------------ tile --
    int64_t m0, m_end, n0;
    const uint8_t* Bp = p.B;
    const float* sBp = p.sB;
    if constexpr (!GROUPED) {
        int id = blockIdx.x;
        const int T = p.tiles_m * p.tiles_n;
        if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);   // contiguous range per XCD
        const int GM = 8;
        const int group = id / (GM * p.tiles_n);
        const int first_m = group * GM;
        const int gsz = min(p.tiles_m - first_m, GM);
        const int in_group = id % (GM * p.tiles_n);
        const int tm = first_m + in_group % gsz;
        const int tn = in_group / gsz;
        m0 = (int64_t)tm * BM;
        m_end = p.M;
        n0 = (int64_t)tn * BN;
    } else {
        // Device-side schedule: exclusive prefix of per-group m-tile counts;
        // virtual tile v -> (group, n-tile, m-tile), m-tile fastest.
        const int64_t v = blockIdx.x;
        int running = 0;
        if (t == 0) s_sel[0] = -1;
        for (int chunk = 0; chunk < p.G; chunk += 256) {
            const int g = chunk + t;
            int cnt = 0;
            int32_t o0 = 0, o1 = 0;
            if (g < p.G) {
                o0 = p.offsets[g];
                o1 = p.offsets[g + 1];
                if (o0 >= 0 && o1 >= o0 && o1 <= p.M) cnt = (o1 - o0 + BM - 1) / BM;
            }
            s_scan[t] = cnt;
            __syncthreads();
            for (int d = 1; d < 256; d <<= 1) {
                int add = (t >= d) ? s_scan[t - d] : 0;
                __syncthreads();
                s_scan[t] += add;
                __syncthreads();
            }
            const int excl = running + s_scan[t] - cnt;
            if (cnt > 0 && v >= (int64_t)excl * p.tiles_n && v < (int64_t)(excl + cnt) * p.tiles_n) {
                s_sel[0] = g;
                s_sel[1] = excl;
            }
            running += s_scan[255];
            __syncthreads();
        }
        __syncthreads();
        const int g = s_sel[0];
        if (g < 0) return;                                    // beyond the last tile
        const int32_t o0 = p.offsets[g], o1 = p.offsets[g + 1];
        const int mt_g = (o1 - o0 + BM - 1) / BM;
        const int64_t local = v - (int64_t)s_sel[1] * p.tiles_n;
        const int tn = (int)(local / mt_g), tm = (int)(local % mt_g);
        m0 = (int64_t)o0 + (int64_t)tm * BM;
        m_end = o1;
        n0 = (int64_t)tn * BN;
        Bp = p.B + (int64_t)g * p.b_group_stride;
        sBp = p.sB + (int64_t)g * p.sb_group_stride;
    }

    // ------------------------------------------------------- loaders --
    const int lrow = t >> 3, lchunk = t & 7;   // 32 rows x 8 chunks of 16 B per pass
    const uint8_t* a_src[4];
    const uint8_t* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t ar = m0 + 32 * i + lrow;
        ar = ar < m_end ? ar : m_end - 1;
        int64_t br = n0 + 32 * i + lrow;
        br = br < p.N ? br : p.N - 1;
        a_src[i] = p.A + ar * p.lda + 16 * lchunk;
        b_src[i] = Bp + br * p.ldb + 16 * lchunk;
    }
    uint4 ra[4], rb[4];
    auto load_tiles = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + (int64_t)kb * BK);
            rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + (int64_t)kb * BK);
        }
    };
    auto store_tiles = [&](int stage) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4*>(&lds[stage][0][(32 * i + lrow) * LDS_STRIDE + 16 * lchunk]) = ra[i];
            *reinterpret_cast<uint4*>(&lds[stage][1][(32 * i + lrow) * LDS_STRIDE + 16 * lchunk]) = rb[i];
        }
    };

    // ------------------------------------------------------- scales ---
    // rows of this lane's accumulators: m = m0 + 64*wm + 32*i + (l & 31)
    int64_t am[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t m = m0 + 64 * wm + 32 * i + (l & 31);
        am[i] = m < m_end ? m : m_end - 1;
    }
    // columns of this lane's accumulators: n = nl + 32*j + 8*q + e
    const int64_t nl = n0 + 64 * wn + 4 * (l >> 5);
    const int64_t nkb = p.K / BK;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    constexpr bool PROMOTE = !(AMODE == FGS_SCALE_TENSOR && BMODE == FGS_SCALE_TENSOR);

    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    for (int64_t kb = 0; kb < nkb; ++kb) {
        const int cur = (int)(kb & 1);
        if (kb + 1 < nkb) load_tiles((int)kb + 1);

        // scales of this K block
        float sa[2] = {1.0f, 1.0f};
        if constexpr (AMODE == FGS_SCALE_TILE_1x128) {
#pragma unroll
            for (int i = 0; i < 2; ++i) sa[i] = p.sA[kb * p.lds_a + am[i]];
        }
        float sb_blk = 1.0f;
        if constexpr (BMODE == FGS_SCALE_BLOCK_128x128) sb_blk = sBp[(n0 / BN) * nkb + kb];

        f32x16 part[2][2];
        if constexpr (PROMOTE) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
        }
        const uint8_t* la = &lds[cur][0][0];
        const uint8_t* lb = &lds[cur][1][0];
        // lane half h reads bytes 32*ks + 16*h .. +15 of its row: the pair of
        // k-steps (2ks, 2ks+1) then covers k = 32*ks .. 32*ks+31 once, with
        // the same k order for A and B
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            f16x8 af[2][2], bf[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                decode16(la + (64 * wm + 32 * i + (l & 31)) * LDS_STRIDE + 32 * ks + 16 * (l >> 5), af[i][0], af[i][1]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                decode16(lb + (64 * wn + 32 * j + (l & 31)) * LDS_STRIDE + 32 * ks + 16 * (l >> 5), bf[j][0], bf[j][1]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if constexpr (PROMOTE)
                            part[i][j] = mfma16(bf[j][h], af[i][h], part[i][j]);
                        else
                            acc[i][j] = mfma16(bf[j][h], af[i][h], acc[i][j]);
                    }
        }

        if constexpr (PROMOTE) {
            float sa_t = 1.0f, sb_t = 1.0f;
            if constexpr (AMODE == FGS_SCALE_TENSOR) sa_t = p.sA[0];
            if constexpr (BMODE == FGS_SCALE_TENSOR) sb_t = sBp[0];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float fa = (AMODE == FGS_SCALE_TENSOR) ? sa_t : sa[i];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if constexpr (BMODE == FGS_SCALE_TILE_1x128) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                int64_t n = nl + 32 * j + 8 * q + e;
                                n = n < p.N ? n : p.N - 1;
                                const float f = fa * sBp[kb * p.lds_b + n];
                                acc[i][j][4 * q + e] = __builtin_fmaf(part[i][j][4 * q + e], f, acc[i][j][4 * q + e]);
                            }
                    } else {
                        const float f = fa * ((BMODE == FGS_SCALE_TENSOR) ? sb_t : sb_blk);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[i][j][r] = __builtin_fmaf(part[i][j][r], f, acc[i][j][r]);
                    }
                }
            }
        }

        if (kb + 1 < nkb) store_tiles(cur ^ 1);
        __syncthreads();
    }

    if constexpr (!PROMOTE) {
        const float f = p.sA[0] * sBp[0];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] *= f;
    }

    // ------------------------------------------------------ epilogue --
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t m = m0 + 64 * wm + 32 * i + (l & 31);
        if (m >= m_end) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + 64 * wn + 32 * j + 8 * q + 4 * (l >> 5);
                if constexpr (OUT_BF16) {
                    uint16_t* C = static_cast<uint16_t*>(p.C) + m * p.ldc + n;
                    uint32_t h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16_rne(acc[i][j][4 * q + e]);
                    if (n + 3 < p.N && ((reinterpret_cast<uintptr_t>(C) & 7) == 0)) {
                        *reinterpret_cast<uint2*>(C) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) C[e] = (uint16_t)h[e];
                    }
                } else {
                    float* C = static_cast<float*>(p.C) + m * p.ldc + n;
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

template <int AMODE, int BMODE, bool GROUPED>
hipError_t launch_modes(const GemmParams& p, bool bf16, dim3 grid, hipStream_t s)
{
    if (bf16)
        hipLaunchKernelGGL((gemm_fp8_kernel<AMODE, BMODE, true, GROUPED>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_fp8_kernel<AMODE, BMODE, false, GROUPED>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <bool GROUPED>
hipError_t dispatch(const GemmParams& p, int amode, int bmode, bool bf16, dim3 grid, hipStream_t s)
{
    if (amode == FGS_SCALE_TILE_1x128) {
        if (bmode == FGS_SCALE_BLOCK_128x128) return launch_modes<FGS_SCALE_TILE_1x128, FGS_SCALE_BLOCK_128x128, GROUPED>(p, bf16, grid, s);
        if constexpr (!GROUPED) {
            if (bmode == FGS_SCALE_TILE_1x128) return launch_modes<FGS_SCALE_TILE_1x128, FGS_SCALE_TILE_1x128, false>(p, bf16, grid, s);
            if (bmode == FGS_SCALE_TENSOR) return launch_modes<FGS_SCALE_TILE_1x128, FGS_SCALE_TENSOR, false>(p, bf16, grid, s);
        }
    } else if constexpr (!GROUPED) {
        if (amode == FGS_SCALE_TENSOR) {
            if (bmode == FGS_SCALE_TENSOR) return launch_modes<FGS_SCALE_TENSOR, FGS_SCALE_TENSOR, false>(p, bf16, grid, s);
            if (bmode == FGS_SCALE_BLOCK_128x128) return launch_modes<FGS_SCALE_TENSOR, FGS_SCALE_BLOCK_128x128, false>(p, bf16, grid, s);
            if (bmode == FGS_SCALE_TILE_1x128) return launch_modes<FGS_SCALE_TENSOR, FGS_SCALE_TILE_1x128, false>(p, bf16, grid, s);
        }
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
    p.lda = a.A.ld;
    p.ldb = a.B.ld;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.lds_a = a.M;
    p.lds_b = a.N;
    p.C = a.C;
    p.ldc = a.ldc;
    p.offsets = a.group_offsets;
    p.G = a.G;
    p.tiles_n = (int32_t)((a.N + BN - 1) / BN);
    if (a.M == 0 || a.N == 0) return hipSuccess;
    if (a.group_offsets) {
        p.b_group_stride = a.N * a.B.ld;
        p.sb_group_stride = ((a.N + BN - 1) / BN) * (a.K / BK);
        const int64_t max_tiles = (a.M + BM - 1) / BM + a.G;
        p.tiles_m = (int32_t)max_tiles;
        dim3 grid((unsigned)(max_tiles * p.tiles_n));
        return dispatch<true>(p, a.A.scale_mode, a.B.scale_mode, a.out_bf16 != 0, grid, stream);
    }
    p.tiles_m = (int32_t)((a.M + BM - 1) / BM);
    dim3 grid((unsigned)((int64_t)p.tiles_m * p.tiles_n));
    return dispatch<false>(p, a.A.scale_mode, a.B.scale_mode, a.out_bf16 != 0, grid, stream);
}

} // namespace fgs
