// util.hip -- workspace fill and the plain streaming copy (the HBM ceiling and the byte-counter
// calibration kernel), gfx950.
#include <algorithm>

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

// The fastest copy measured on MI355X (7.5 GB each way: 6.70-6.76 TB/s against 6.64-6.68 for
// copy_vec_kernel): one persistent workgroup per CU, 64 KiB units (16 vectors per thread) taken
// in order from a counter, two register buffers -- the next unit is loaded before the current
// one is stored. Two workgroups per CU, or a static split of the units, measured slower
// (6.0 and 4.9-5.2 TB/s). units = ceil(nv / kPersistVecs); the counter starts at zero.
constexpr int kPersistVec = 16;
constexpr int64_t kPersistVecs = (int64_t)kBlock * kPersistVec;

__global__ __launch_bounds__(kBlock) void copy_persist_kernel(const f4* __restrict__ s,
                                                              f4* __restrict__ d, int64_t nv,
                                                              uint32_t* counter)
{
    __shared__ uint32_t next;
    const int64_t units = (nv + kPersistVecs - 1) / kPersistVecs;
    auto grab = [&]() -> int64_t {
        if (threadIdx.x == 0)
            next = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int64_t u = next;
        __syncthreads();
        return u;
    };
    // whole units take unconditional accesses (a load under a branch is waited for at the
    // branch's end, which would serialize the unit's 16 loads); only a ragged last unit checks
    auto load = [&](f4 (&r)[kPersistVec], int64_t u) {
        const int64_t i0 = u * kPersistVecs + threadIdx.x;
        if ((u + 1) * kPersistVecs <= nv) {
#pragma unroll
            for (int j = 0; j < kPersistVec; ++j) r[j] = ld_stream(s + i0 + j * kBlock);
        } else {
#pragma unroll
            for (int j = 0; j < kPersistVec; ++j)
                if (i0 + j * kBlock < nv) r[j] = ld_stream(s + i0 + j * kBlock);
        }
    };
    auto store = [&](const f4 (&r)[kPersistVec], int64_t u) {
        const int64_t i0 = u * kPersistVecs + threadIdx.x;
        if ((u + 1) * kPersistVecs <= nv) {
#pragma unroll
            for (int j = 0; j < kPersistVec; ++j) st_stream(d + i0 + j * kBlock, r[j]);
        } else {
#pragma unroll
            for (int j = 0; j < kPersistVec; ++j)
                if (i0 + j * kBlock < nv) st_stream(d + i0 + j * kBlock, r[j]);
        }
    };
    f4 A[kPersistVec], B[kPersistVec];
    int64_t ua = grab();
    if (ua >= units) return;
    load(A, ua);
    for (;;) {
        const int64_t ub = grab();
        if (ub < units) load(B, ub);
        store(A, ua);
        if (ub >= units) return;
        ua = grab();
        if (ua < units) load(A, ua);
        store(B, ub);
        if (ua >= units) return;
    }
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

hipError_t launch_stream_copy_persistent(const float* src, float* dst, int64_t n, void* counter,
                                         hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t nv = n / 4;  // the caller checked 16-byte alignment and n % 4 == 0
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if ((e = launch_fill_zero(counter, 4, stream)) != hipSuccess) return e;
    const int64_t units = (nv + kPersistVecs - 1) / kPersistVecs;
    const int64_t grid = std::min<int64_t>(units, cus > 0 ? cus : 256);
    copy_persist_kernel<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(
        reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst), nv, static_cast<uint32_t*>(counter));
    return hipGetLastError();
}

}  // namespace nr
