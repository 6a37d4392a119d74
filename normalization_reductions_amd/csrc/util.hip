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

// One 16-byte vector per thread, one 4 KiB chunk per workgroup, a one-shot grid. Workgroups
// are dealt to the XCDs round-robin, so chunk b is remapped to let each XCD stream its own
// contiguous eighth of the buffer (measured the fastest copy pattern on MI355X: a fine-grained
// stream per XCD beats persistent grids and large per-workgroup chunks).
__global__ __launch_bounds__(kBlock) void copy_vec_kernel(const f4* __restrict__ s,
                                                          f4* __restrict__ d, int64_t nv,
                                                          int64_t nchunks)
{
    int64_t b = blockIdx.x;
    const int64_t n8 = nchunks / 8 * 8;
    if (b < n8) b = (b % 8) * (n8 / 8) + b / 8;
    const int64_t i = b * kBlock + threadIdx.x;
    if (i < nv) st_stream(d + i, ld_stream(s + i));
}

__global__ __launch_bounds__(kBlock) void copy_scalar_kernel(const float* __restrict__ s,
                                                             float* __restrict__ d, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        d[i] = s[i];
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
    if (vec && (n / 4 + kBlock - 1) / kBlock <= 0x7fffffffLL) {
        const int64_t nv = n / 4;
        const int64_t nchunks = (nv + kBlock - 1) / kBlock;
        copy_vec_kernel<<<dim3((unsigned)nchunks), dim3(kBlock), 0, stream>>>(
            reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst), nv, nchunks);
    } else {
        int64_t grid = (n + kBlock - 1) / kBlock;
        if (grid > 65536) grid = 65536;
        copy_scalar_kernel<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(src, dst, n);
    }
    return hipGetLastError();
}

}  // namespace nr
