// quant_e4m3.hip -- online FP32-scaled E4M3 quantization on gfx950.
//
// "Can you explain the role of FP8 precision in DeepSeek-V3 training",
// sections "Fine-grained quantization" (activations in 1x128 tiles, weights
// in 128x128 blocks, each with its own scale) and "Online quantization"
// (the scale is derived from the current tile/block amax); "Accelerating FP8
// training performance with the NVIDIA NeMo framework" (per-tensor current
// scaling).  The rule: scale = fl32(amax / 448), code = E4M3_RNE_SAT(x / s).
//
// One workgroup (256 threads, 4 waves) owns a 128 x 128 block of the BF16
// source.  Thread t (wave w, lane l) holds an 8 x 8 sub-block:
//   column group cg = l & 15         -> source columns c0 + 8*cg .. +7
//   row group    rg = 4*w + (l >> 4) -> source rows    r0 + 8*rg .. +7
// Each of its eight 16-byte loads reads row r0 + 8*rg + u; the 16 lanes of a
// DPP row read one 256-byte contiguous row segment.  From the one read the
// kernel emits the row-wise codes (1x128 tiles = one row of the block, or
// the block / tensor scale) and the column-wise codes (128x1 tiles along the
// source rows, the wgrad operand, or the transposed block/tensor codes),
// the latter transposed through LDS so every store is a full 128-byte row.
#include <mutex>
#include <type_traits>

#include "fgs_device.h"
#include "fgs_internal.h"

namespace fgs {

// Scratch of the allocation-free per-tensor quantization
// (fgs_quantize_blockwise_noalloc): the amax pass's per-workgroup partials,
// one 4-byte slot per amax workgroup.  Every GPU the library runs on holds
// its own copy until the process ends.  Host code never passes this name to
// a kernel (on the host it is a stand-in, not a device address): the
// per-device address comes from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = 4 * 1024;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

namespace {

constexpr int TB = 128;        // block edge
constexpr int TPAD = 16;       // LDS row padding of the transposed code tile

__device__ __forceinline__ uint32_t abs_max8(const uint4& v)
{
    uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
    uint32_t c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
    uint32_t m0 = max(a & 0xFFFFu, a >> 16), m1 = max(b & 0xFFFFu, b >> 16);
    uint32_t m2 = max(c & 0xFFFFu, c >> 16), m3 = max(d & 0xFFFFu, d >> 16);
    return max(max(m0, m1), max(m2, m3));
}

// |BF16| bits of element j (0..7) of an 8-element vector
__device__ __forceinline__ uint32_t abs_elem(const uint4& v, int j)
{
    uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
    return ((j & 1) ? (w >> 16) : w) & 0x7FFFu;
}

__device__ __forceinline__ uint32_t raw_elem(const uint4& v, int j)
{
    uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// FP32 value of element j (0..7) of an 8-element BF16 vector (exact)
__device__ __forceinline__ uint32_t val_bits(const uint4& v, int j)
{
    const uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
    return (j & 1) ? (w & 0xFFFF0000u) : (w << 16);
}

// Codes of 8 values (FP32 bit patterns of BF16 numbers) of one block.
// SPECIAL: the block may be non-finite or pre-scaled (per-lane tests);
// without it the caller guarantees neither (the common, branch-free form).
template <bool SPECIAL>
__device__ __forceinline__ uint2 quant8_vals(const uint32_t xb[8], const E4M3Block& b)
{
    if constexpr (SPECIAL) {
        if (b.nan) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    }
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = SPECIAL ? e4m3_quotient_bits(xb[j], b) : e4m3_quotient_plain(xb[j], b);
    return make_uint2(e4m3_pack4(q[0], q[1], q[2], q[3]), e4m3_pack4(q[4], q[5], q[6], q[7]));
}

template <bool SPECIAL>
__device__ __forceinline__ uint2 quant8(const uint4& v, const E4M3Block& b)
{
    uint32_t xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xb[j] = val_bits(v, j);
    return quant8_vals<SPECIAL>(xb, b);
}

// true on every lane when any lane of the wave passes true: a wave-uniform
// branch condition
__device__ __forceinline__ bool wave_any(bool p)
{
    return __builtin_amdgcn_ballot_w64(p) != 0;
}

// SwiGLU of one BF16 (gate, up) pair: h = silu(g) * u in FP32, rounded to
// BF16 (nearest even, by the hardware converter).  The logistic factor is
// formed from exp(-|g|) <= 1 on both sides of zero, so it never overflows:
// 1 / (1 + e) for g >= 0, e / (1 + e) for g < 0.
__device__ __forceinline__ uint32_t swiglu_bf16_bits(uint32_t gb, uint32_t ub)
{
    const float g = as_f32(gb), u = as_f32(ub);
    const float e = expf(-__builtin_fabsf(g));
    const float d = 1.0f + e;
    const float sig = (g >= 0.0f) ? 1.0f / d : e / d;
    const float h = (g * sig) * u;
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)h);
}

// Eight SwiGLU activations from the gate and up vectors of one row.
__device__ __forceinline__ uint4 swiglu8(const uint4& g, const uint4& u)
{
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = swiglu_bf16_bits(val_bits(g, j), val_bits(u, j));
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// GROUPED (TILE mode only): the rows are split into groups (MoE experts,
// rows offsets[g] .. offsets[g+1]-1), and the column-wise tiles run along the
// rows of one group only.  Group g's transposed codes take the 128-column
// blocks kb_g = floor(offsets[g] / 128) + g .. kb_g + ceil(M_g / 128) - 1 of
// qT (row stride ldqT) and the same rows of scalesT; those blocks never
// overlap for non-decreasing offsets, so no scan over the groups is needed.
// Workgroup (blockIdx.x = column block, blockIdx.y = block j) finds the group
// that owns block j; rows past the group's end read as zero (zero codes in
// qT, no effect on the amax).  The column blocks of one row block are
// launched side by side, so the 256-byte segments of a row are read together
// (measured 2-10% faster than row blocks side by side).  With row_index, logical row t is source row
// row_index[t] of x (the MoE dispatch gather, fused so the permuted BF16
// copy is never written); an index outside [0, src_rows) reads as zeros.
// SWIGLU (GROUPED only): x holds a gate/up GEMM output [rows x 2*cols] and
// the quantized matrix is its SwiGLU activation, computed on the load (with
// its BF16 values optionally stored to h_out [rows x cols]), so the
// activation is never written and read back before the down projection.
// Occupancy: the 1x128 kernels hold sixteen block scales per thread; asked
// for six (dense) or five (grouped) resident workgroups per CU they fit 80 or
// 96 VGPRs without spilling (101 unconstrained: four workgroups).  The other
// modes use 49.
template <int MODE, bool GROUPED, bool SWIGLU = false>   // MODE: FGS_SCALE_TILE_1x128 | FGS_SCALE_BLOCK_128x128 | FGS_SCALE_TENSOR
__global__ __launch_bounds__(256, GROUPED ? 5 : 6) void quant_e4m3_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q, float* __restrict__ scales,
    uint8_t* __restrict__ qT, float* __restrict__ scalesT,
    const uint32_t* __restrict__ tensor_amax, int32_t n_amax,
    const int32_t* __restrict__ offsets, int32_t G, int64_t ldqT,
    const int32_t* __restrict__ row_index, int64_t src_rows, uint16_t* __restrict__ h_out)
{
    static_assert(!GROUPED || MODE == FGS_SCALE_TILE_1x128, "groups take 1x128 tiles");
    static_assert(!SWIGLU || GROUPED, "the SwiGLU prologue belongs to the grouped quantizer");
    __shared__ uint32_t red[4][TB];
    __shared__ __align__(16) uint8_t tbuf[TB][TB + TPAD];
    __shared__ int s_group;

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = l & 15, rg = 4 * w + (l >> 4);
    // r0: first source row; live: rows of this block that exist (from r0);
    // tc: first column of qT; tb: row of scalesT; ldt: row stride of qT
    int64_t r0, c0, live, tc, tb, ldt;
    if constexpr (!GROUPED) {
        r0 = (int64_t)blockIdx.y * TB;
        c0 = (int64_t)blockIdx.x * TB;
        live = rows - r0;
        tc = r0;
        tb = blockIdx.y;
        ldt = rows;
    } else {
        const int64_t j = blockIdx.y;
        if (t == 0) s_group = -1;
        __syncthreads();
        for (int g = t; g < G; g += 256) {
            const int32_t o0 = offsets[g], o1 = offsets[g + 1];
            if (o0 >= 0 && o1 >= o0 && (int64_t)o1 <= rows) {
                const int64_t kb = (int64_t)(o0 >> 7) + g;
                if (j >= kb && j < kb + (o1 - o0 + TB - 1) / TB) s_group = g;
            }
        }
        __syncthreads();
        const int g = s_group;
        if (g < 0) return;                       // a block no group owns
        const int32_t o0 = offsets[g], o1 = offsets[g + 1];
        r0 = (int64_t)o0 + (j - ((int64_t)(o0 >> 7) + g)) * TB;
        c0 = (int64_t)blockIdx.x * TB;
        live = (int64_t)o1 - r0;
        tc = j * TB;
        tb = j;
        ldt = ldqT;
    }
    const int64_t col = c0 + 8 * cg;
    const bool col_ok = col < cols;

    // per-thread base of row 8*rg (u * stride is wave-uniform)
    const uint16_t* const x_base = x + (r0 + 8 * rg) * ldx + col;
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t row = r0 + 8 * rg + u;
        bool ok = col_ok && 8 * rg + u < live;
        int64_t src = row;
        if constexpr (GROUPED) {
            if (row_index && ok) {
                src = row_index[row];
                ok = src >= 0 && src < src_rows;
            }
        }
        if constexpr (SWIGLU) {
            if (ok) {
                const uint16_t* xr = x + src * ldx + col;
                v[u] = swiglu8(load_nt16(xr), load_nt16(xr + cols));
                if (h_out) *reinterpret_cast<uint4*>(h_out + row * cols + col) = v[u];
            } else {
                v[u] = make_uint4(0, 0, 0, 0);
            }
        } else {
            // a dispatch gather reads each token's row several times (top-k
            // routing), so it keeps the caches; other rows are read once
            if (ok)
                v[u] = (GROUPED && row_index) ? *reinterpret_cast<const uint4*>(x + src * ldx + col)
                                              : load_nt16(x_base + u * ldx);
            else
                v[u] = make_uint4(0, 0, 0, 0);
        }
    }

    // ---------------- shared (block / tensor) scale --------------------
    E4M3Block shared_b;
    if constexpr (MODE == FGS_SCALE_BLOCK_128x128) {
        uint32_t m = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = max(m, abs_max8(v[u]));
        m = max_xor32(max_xor16(max_lanes16(m)));
        if (l == 0) red[w][0] = m;
        __syncthreads();
        m = max(max(red[0][0], red[1][0]), max(red[2][0], red[3][0]));
        shared_b = e4m3_block_from_amax_bits(m);
        if (t == 0) {
            if (q) scales[blockIdx.y * ((cols + TB - 1) / TB) + blockIdx.x] = shared_b.s;
            if (qT) scalesT[blockIdx.x * ((rows + TB - 1) / TB) + blockIdx.y] = shared_b.s;
        }
    } else if constexpr (MODE == FGS_SCALE_TENSOR) {
        // the tensor amax: the max of the amax pass's per-workgroup partials
        // (read after this block's own loads are in flight)
        uint32_t m = 0;
        for (int i = t; i < n_amax; i += 256) m = max(m, tensor_amax[i]);
        m = max_xor32(max_xor16(max_lanes16(m)));
        if (l == 0) red[w][0] = m;
        __syncthreads();
        m = max(max(red[0][0], red[1][0]), max(red[2][0], red[3][0]));
        shared_b = e4m3_block_from_amax_bits(m);
        if (t == 0 && blockIdx.x == 0 && blockIdx.y == 0) {
            if (scales) scales[0] = shared_b.s;
            if (scalesT) scalesT[0] = shared_b.s;
        }
    }

    // ---------------- row-wise output ---------------------------------
    if (q) {
        float srow[8];
        uint32_t mrow[8];
        bool special = false;
        if constexpr (MODE == FGS_SCALE_TILE_1x128) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                mrow[u] = max_lanes16(abs_max8(v[u]));
                special |= e4m3_block_special(mrow[u]);
            }
        } else {
            special = shared_b.nan || shared_b.k != 1.0f;
        }
        uint8_t* const q_base = q + (r0 + 8 * rg) * cols + col;
        auto emit = [&](auto special_c) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                E4M3Block b;
                if constexpr (MODE == FGS_SCALE_TILE_1x128) {
                    b = decltype(special_c)::value ? e4m3_block_from_amax_bits(mrow[u])
                                                   : e4m3_block_plain(mrow[u]);
                    srow[u] = b.s;
                } else {
                    b = shared_b;
                }
                const uint2 codes = quant8<decltype(special_c)::value>(v[u], b);
                if (col_ok && 8 * rg + u < live) {
                    uint8_t* dst = q_base + u * cols;
                    // non-temporal stores measured faster for the grouped
                    // (MoE) layout (plain stores there cost the next GEMM
                    // more than they save) and slower for the dense one
                    if constexpr (GROUPED) store_nt8(dst, codes);
                    else *reinterpret_cast<uint2*>(dst) = codes;
                }
            }
        };
        if (wave_any(special)) emit(std::true_type{});
        else emit(std::false_type{});
        if constexpr (MODE == FGS_SCALE_TILE_1x128) {
            if (cg == 0) {
                float* dst = scales + (c0 / TB) * rows + r0 + 8 * rg;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (8 * rg + u < live) dst[u] = srow[u];
            }
        }
    }

    // ---------------- column-wise (transposed) output ------------------
    if (qT) {
        uint32_t mcol[8];     // 1x128 mode: |BF16| amax bits of columns 8*cg + j
        bool special = false;
        if constexpr (MODE == FGS_SCALE_TILE_1x128) {
            uint32_t cm[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t m = 0;
#pragma unroll
                for (int u = 0; u < 8; ++u) m = max(m, abs_elem(v[u], j));
                cm[j] = max_xor32(max_xor16(m));
            }
            if ((l >> 4) == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) red[w][8 * cg + j] = cm[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = 8 * cg + j;
                mcol[j] = max(max(red[0][c], red[1][c]), max(red[2][c], red[3][c]));
                special |= e4m3_block_special(mcol[j]);
            }
        } else {
            special = shared_b.nan || shared_b.k != 1.0f;
        }
        // codes of column j, rows 8*rg .. 8*rg+7 -> 8 contiguous bytes of qT
        // one column block's constants live at a time (eight at once cost
        // the 1x128 kernel occupancy)
        auto emit = [&](auto special_c) {
            constexpr bool SPECIAL = decltype(special_c)::value;
            const bool scale_writer = w == 0 && (l >> 4) == 0 && col_ok;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                E4M3Block b;
                if constexpr (MODE == FGS_SCALE_TILE_1x128) {
                    b = SPECIAL ? e4m3_block_from_amax_bits(mcol[j]) : e4m3_block_plain(mcol[j]);
                    if (scale_writer) scalesT[tb * cols + col + j] = b.s;
                } else {
                    b = shared_b;
                }
                uint32_t xb[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) xb[u] = val_bits(v[u], j);
                *reinterpret_cast<uint2*>(&tbuf[8 * cg + j][8 * rg]) = quant8_vals<SPECIAL>(xb, b);
            }
        };
        if (wave_any(special)) emit(std::true_type{});
        else emit(std::false_type{});
        __syncthreads();
        // 8 lanes write one 128-byte row of qT
        const int chunk = t & 7;
        uint8_t* const qT_base = qT + (c0 + (t >> 3)) * ldt + tc + 16 * chunk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int trow = 32 * i + (t >> 3);
            if (c0 + trow < cols) {
                uint4 d = *reinterpret_cast<const uint4*>(&tbuf[trow][16 * chunk]);
                uint8_t* const dst = qT_base + 32 * i * ldt;
                if constexpr (GROUPED) store_nt16(dst, d);
                else *reinterpret_cast<uint4*>(dst) = d;
            }
        }
    }
}

// Tensor amax (|BF16| bits) of a 128 x 128-block grid, as one partial per
// workgroup (out[blockIdx.x]; the cast kernel takes the max of the
// gridDim.x partials, so no same-address atomics and no clearing pass):
// persistent over the blocks with stride gridDim.x, the next block's rows loaded before the
// current ones are reduced.
__global__ __launch_bounds__(256) void amax_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    int64_t nbr, int64_t nbc, uint32_t* __restrict__ out)
{
    __shared__ uint32_t red[4];
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int cg = l & 15, rg = 4 * w + (l >> 4);
    const int64_t nblk = nbr * nbc;
    auto load = [&](int64_t blk, uint4 v[8]) {
        const int64_t r0 = (blk / nbc) * TB, col = (blk % nbc) * TB + 8 * cg;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t row = r0 + 8 * rg + u;
            v[u] = (col < cols && row < rows) ? load_nt16(x + row * ldx + col)
                                              : make_uint4(0, 0, 0, 0);
        }
    };
    uint32_t m = 0;
    int64_t blk = blockIdx.x;
    uint4 v[8];
    if (blk < nblk) load(blk, v);
    while (blk < nblk) {
        const int64_t next = blk + gridDim.x;
        uint4 vn[8];
        if (next < nblk) load(next, vn);
#pragma unroll
        for (int u = 0; u < 8; ++u) m = max(m, abs_max8(v[u]));
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = vn[u];
        blk = next;
    }
    m = max_xor32(max_xor16(max_lanes16(m)));
    if (l == 0) red[w] = m;
    __syncthreads();
    if (t == 0) out[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Tensor amax of a contiguous tensor (ldx == cols), read as a flat array of
// n16 16-byte chunks: persistent, consecutive lanes on consecutive chunks
// (each wave-instruction reads 1 KiB of contiguous memory), eight
// non-temporal loads in flight per thread; one partial per workgroup, as
// amax_bf16_kernel.  Every index touched is below n16: the unrolled body
// runs only while its last index is.
__global__ __launch_bounds__(256) void amax_bf16_flat_kernel(const uint16_t* __restrict__ x, int64_t n16,
                                                             uint32_t* __restrict__ out)
{
    constexpr int UNROLL = 8;
    __shared__ uint32_t red[4];
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + t;
    uint32_t m = 0;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = load_nt16(x + 8 * (i + u * stride));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) m = max(m, abs_max8(v[u]));
    }
    for (; i < n16; i += stride) m = max(m, abs_max8(load_nt16(x + 8 * i)));
    m = max_xor32(max_xor16(max_lanes16(m)));
    if (l == 0) red[w] = m;
    __syncthreads();
    if (t == 0) out[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

} // namespace

hipError_t launch_quant_e4m3(const QuantE4M3Args& a, hipStream_t stream)
{
    const int64_t nbr = (a.rows + TB - 1) / TB, nbc = (a.cols + TB - 1) / TB;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    dim3 grid((unsigned)nbc, (unsigned)nbr), block(256);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    switch (a.mode) {
    case FGS_SCALE_TILE_1x128:
        hipLaunchKernelGGL((quant_e4m3_kernel<FGS_SCALE_TILE_1x128, false>), grid, block, 0, stream,
                           x, a.rows, a.cols, a.ldx, a.q, a.scales, a.qT, a.scalesT, nullptr, 0, nullptr, 0, 0, nullptr, 0, nullptr);
        break;
    case FGS_SCALE_BLOCK_128x128:
        hipLaunchKernelGGL((quant_e4m3_kernel<FGS_SCALE_BLOCK_128x128, false>), grid, block, 0, stream,
                           x, a.rows, a.cols, a.ldx, a.q, a.scales, a.qT, a.scalesT, nullptr, 0, nullptr, 0, 0, nullptr, 0, nullptr);
        break;
    case FGS_SCALE_TENSOR: {
        // amax workgroups: two per compute unit (each keeps two blocks of
        // loads in flight), at most one per 4-byte workspace slot
        uint32_t* amax = static_cast<uint32_t*>(a.workspace);
        const int64_t slots = (int64_t)(a.workspace_bytes / 4);
        int64_t g;
        if (a.ldx == a.cols) {
            // contiguous: stream it as one flat array, one workgroup per
            // compute unit (the read ceiling's configuration)
            const int64_t n16 = a.rows * a.cols / 8;
            g = (n16 + 255) / 256;
            const int64_t cap = (int64_t)device_cus();
            if (g > cap) g = cap;
            if (g > slots) g = slots;
            hipLaunchKernelGGL(amax_bf16_flat_kernel, dim3((unsigned)g), block, 0, stream, x, n16, amax);
        } else {
            g = nbr * nbc;
            const int64_t cap = (int64_t)device_cus() * 2;
            if (g > cap) g = cap;
            if (g > slots) g = slots;
            hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)g), block, 0, stream,
                               x, a.rows, a.cols, a.ldx, nbr, nbc, amax);
        }
        hipLaunchKernelGGL((quant_e4m3_kernel<FGS_SCALE_TENSOR, false>), grid, block, 0, stream,
                           x, a.rows, a.cols, a.ldx, a.q, a.scales, a.qT, a.scalesT, amax, (int32_t)g,
                           nullptr, 0, 0, nullptr, 0, nullptr);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Device address of `scratch` on the current device, resolved once per
// device (with that device current) and kept.
hipError_t quant_scratch(void** ptr, size_t* bytes)
{
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static void* addr[kMaxDevices];
    static hipError_t status[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] {
        void* p = nullptr;
        status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        addr[dev] = p;
    });
    if (status[dev] != hipSuccess) return status[dev];
    *ptr = addr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

hipError_t launch_quant_grouped_colwise(const QuantGroupedArgs& a, hipStream_t stream)
{
    // every group owns at most floor(rows / 128) + G blocks in total
    const int64_t nblk = a.rows / TB + a.G, nbc = (a.cols + TB - 1) / TB;
    if (a.G == 0 || a.rows == 0 || nbc == 0) return hipSuccess;
    const dim3 grid((unsigned)nbc, (unsigned)nblk);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (a.swiglu)
        hipLaunchKernelGGL((quant_e4m3_kernel<FGS_SCALE_TILE_1x128, true, true>), grid, dim3(256), 0, stream,
                           x, a.rows, a.cols, a.ldx, a.q, a.scales, a.qT, a.scalesT, nullptr, 0, a.group_offsets,
                           a.G, a.ldqT, a.row_index, a.src_rows, a.h_out);
    else
        hipLaunchKernelGGL((quant_e4m3_kernel<FGS_SCALE_TILE_1x128, true>), grid, dim3(256), 0, stream,
                           x, a.rows, a.cols, a.ldx, a.q, a.scales, a.qT, a.scalesT, nullptr, 0, a.group_offsets,
                           a.G, a.ldqT, a.row_index, a.src_rows, nullptr);
    return hipGetLastError();
}

} // namespace fgs
