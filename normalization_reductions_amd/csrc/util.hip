// util.hip -- workspace fill and the plain streaming copy (the HBM ceiling and the byte-counter
// calibration kernel), gfx950.
#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(uint32_t* p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * kBlock)
        p[i] = 0u;
}

__global__ __launch_bounds__(kBlock) void fill_zero_bytes_kernel(unsigned char* p, int64_t n)
{
    const int64_t i = threadIdx.x;
    if (i < n) p[i] = 0;
}

// Each thread moves 4 x 16 bytes per iteration; the grid strides over the whole buffer.
__global__ __launch_bounds__(kBlock) void copy_vec_kernel(const f4* __restrict__ s,
                                                          f4* __restrict__ d, int64_t nv)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock * 4;
    for (int64_t i0 = (int64_t)blockIdx.x * kBlock * 4 + threadIdx.x; i0 < nv; i0 += stride) {
        f4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = i0 + j * kBlock;
            if (i < nv) v[j] = ld_stream(s + i);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = i0 + j * kBlock;
            if (i < nv) st_stream(d + i, v[j]);
        }
    }
}

__global__ __launch_bounds__(kBlock) void copy_scalar_kernel(const float* __restrict__ s,
                                                             float* __restrict__ d, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        d[i] = s[i];
}

int cu_count()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 256;
    return cus > 0 ? cus : 256;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream)
{
    const int64_t words = (int64_t)(bytes / 4);
    if (words > 0) {
        int64_t grid = (words + kBlock - 1) / kBlock;
        if (grid > 4096) grid = 4096;
        fill_zero_kernel<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(
            static_cast<uint32_t*>(p), words);
    }
    const int64_t tail = (int64_t)(bytes & 3);
    if (tail)
        fill_zero_bytes_kernel<<<1, kBlock, 0, stream>>>(static_cast<unsigned char*>(p) + words * 4,
                                                         tail);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const float* src, float* dst, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0 &&
                     (n & 3) == 0;
    if (vec) {
        const int64_t nv = n / 4;
        int64_t grid = (nv + kBlock * 4 - 1) / (kBlock * 4);
        const int64_t cap = (int64_t)cu_count() * 8;  // a few resident waves per SIMD, persistent
        if (grid > cap) grid = cap;
        copy_vec_kernel<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(
            reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst), nv);
    } else {
        int64_t grid = (n + kBlock - 1) / kBlock;
        if (grid > 65536) grid = 65536;
        copy_scalar_kernel<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(src, dst, n);
    }
    return hipGetLastError();
}

}  // namespace nr
