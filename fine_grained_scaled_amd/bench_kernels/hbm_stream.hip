// hbm_stream.hip -- HBM ceilings for the quantizers' roofline: a streaming
// read (every byte of a buffer loaded once, reduced to one word per
// workgroup) and a streaming copy.  Built into libfgs_hbm.so, which only the
// benchmark loads; it is not part of the product's C ABI.
//
// Both kernels are persistent over the buffer: the grid holds a fixed number
// of workgroups per compute unit, each thread keeps UNROLL 16-byte loads in
// flight, and consecutive lanes touch consecutive 16-byte chunks, so every
// wave-instruction covers 1 KiB of contiguous memory.  Variants differ in
// the unroll depth and in non-temporal access; the benchmark takes the
// best of them as the ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int THREADS = 256;

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p)
{
    if constexpr (NT) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        return make_uint4(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                          __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3));
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st16(uint4* p, const uint4& v)
{
    if constexpr (NT) {
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
        __builtin_nontemporal_store(v.x, q);
        __builtin_nontemporal_store(v.y, q + 1);
        __builtin_nontemporal_store(v.z, q + 2);
        __builtin_nontemporal_store(v.w, q + 3);
    } else {
        *p = v;
    }
}

// Every index touched is below n16: the unrolled body runs only while its
// last index is, and the tail loop covers the rest one load at a time.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(THREADS) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                              uint32_t* __restrict__ out)
{
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = ld16<NT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = ld16<NT>(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[THREADS];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int d = THREADS / 2; d > 0; d >>= 1) {
        if ((int)threadIdx.x < d) red[threadIdx.x] ^= red[threadIdx.x + d];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

template <int UNROLL, bool NT>
__global__ __launch_bounds__(THREADS) void stream_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                              int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = ld16<NT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) st16<NT>(dst + i + u * stride, v[u]);
    }
    for (; i < n16; i += stride) st16<NT>(dst + i, ld16<NT>(src + i));
}

int grid_for(int per_cu)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    }
    return cus * per_cu;
}

} // namespace

extern "C" {

// Number of kernel variants: variant v unrolls 4 << (v % 3) loads per thread
// (4, 8 or 16) and uses non-temporal loads and stores when v >= 3.
int fgs_hbm_variants(void) { return 6; }

// Workgroups the kernels launch with `per_cu` workgroups per compute unit:
// the size of the read kernel's `out` buffer (uint32 words).
int fgs_hbm_read_grid(int per_cu) { return grid_for(per_cu); }

// Reads `bytes` (a multiple of 16, src 16-byte aligned) once; out: device
// uint32 [fgs_hbm_read_grid(per_cu)].  Returns 0 or a hipError_t.
int fgs_hbm_read(const void* src, int64_t bytes, uint32_t* out, int per_cu, int variant, void* stream)
{
    if (bytes <= 0 || bytes % 16 || per_cu < 1 || per_cu > 32 || variant < 0 || variant >= 6)
        return (int)hipErrorInvalidValue;
    const dim3 g(grid_for(per_cu)), b(THREADS);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* x = static_cast<const uint4*>(src);
    switch (variant) {
    case 0: hipLaunchKernelGGL((stream_read_kernel<4, false>), g, b, 0, s, x, bytes / 16, out); break;
    case 1: hipLaunchKernelGGL((stream_read_kernel<8, false>), g, b, 0, s, x, bytes / 16, out); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<16, false>), g, b, 0, s, x, bytes / 16, out); break;
    case 3: hipLaunchKernelGGL((stream_read_kernel<4, true>), g, b, 0, s, x, bytes / 16, out); break;
    case 4: hipLaunchKernelGGL((stream_read_kernel<8, true>), g, b, 0, s, x, bytes / 16, out); break;
    default: hipLaunchKernelGGL((stream_read_kernel<16, true>), g, b, 0, s, x, bytes / 16, out); break;
    }
    return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned).
int fgs_hbm_copy(void* dst, const void* src, int64_t bytes, int per_cu, int variant, void* stream)
{
    if (bytes <= 0 || bytes % 16 || per_cu < 1 || per_cu > 32 || variant < 0 || variant >= 6)
        return (int)hipErrorInvalidValue;
    const dim3 g(grid_for(per_cu)), b(THREADS);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* x = static_cast<const uint4*>(src);
    uint4* y = static_cast<uint4*>(dst);
    switch (variant) {
    case 0: hipLaunchKernelGGL((stream_copy_kernel<4, false>), g, b, 0, s, x, y, bytes / 16); break;
    case 1: hipLaunchKernelGGL((stream_copy_kernel<8, false>), g, b, 0, s, x, y, bytes / 16); break;
    case 2: hipLaunchKernelGGL((stream_copy_kernel<16, false>), g, b, 0, s, x, y, bytes / 16); break;
    case 3: hipLaunchKernelGGL((stream_copy_kernel<4, true>), g, b, 0, s, x, y, bytes / 16); break;
    case 4: hipLaunchKernelGGL((stream_copy_kernel<8, true>), g, b, 0, s, x, y, bytes / 16); break;
    default: hipLaunchKernelGGL((stream_copy_kernel<16, true>), g, b, 0, s, x, y, bytes / 16); break;
    }
    return (int)hipGetLastError();
}

} // extern "C"
