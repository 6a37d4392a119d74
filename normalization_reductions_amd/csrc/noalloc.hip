// noalloc.hip -- instance norm for callers that cannot allocate device memory (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc), gfx950.
//
// inorm_forward_noalloc runs inorm_forward with its workspace in `scratch`, a device array of
// kNoAllocScratchBytes that the library holds on every GPU it runs on until the process ends.
// In host code the name `scratch` only stands in for the array: its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) on the entry point's
// first call there, and that address is what the kernels receive. Every call on one GPU shares
// that GPU's array: calls that overlap on one GPU (two streams, or two threads without
// ordering) race. Whatever must start at zero (the exchange counter and slots) is cleared by a
// fill kernel on the call's stream, as for any workspace; the array's sticky error word keeps
// the last flags raised (zero at load, never cleared by these calls).
#include <mutex>

#include "internal.hpp"
#include "normred.h"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;  // covers x[112,64,512,512] (3.7 MiB)
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

}  // namespace

extern "C" __attribute__((visibility("default"))) nr_status inorm_forward_noalloc(
    const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps, const float* gamma,
    const float* beta, float* save_mean, float* save_invstd, hipStream_t stream)
{
    static const char* fn = "inorm_forward_noalloc";
    const size_t need = inorm_workspace_size(N, C, S);
    if (need == 0)  // sizes inorm_forward rejects: let it report them
        return inorm_forward(x, y, N, C, S, eps, gamma, beta, save_mean, save_invstd, nullptr, 0,
                             stream);
    if (need > kNoAllocScratchBytes)
        return nr::set_error(NR_ERR_WORKSPACE,
                             "%s: x[%lld,%lld,%lld] needs %zu bytes of workspace; the "
                             "no-allocation entry point holds %zu (use inorm_forward with a "
                             "workspace of your own)",
                             fn, (long long)N, (long long)C, (long long)S, need, kNoAllocScratchBytes);
    if (N * C == 0)  // empty batch: a no-op that touches no device
        return inorm_forward(x, y, N, C, S, eps, gamma, beta, save_mean, save_invstd, nullptr, 0,
                             stream);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return nr::set_error(NR_ERR_HIP, "%s: hipGetDevice: HIP error %d (%s)", fn, (int)e,
                             hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return nr::set_error(NR_ERR_UNSUPPORTED, "%s: device %d beyond the %d this entry point serves",
                             fn, dev, kMaxDevices);
    std::call_once(g_scratch_once[dev], [dev] {
        g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev])
        return nr::set_error(NR_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: HIP error %d (%s)",
                             fn, dev, (int)g_scratch_err[dev], hipGetErrorString(g_scratch_err[dev]));
    return inorm_forward(x, y, N, C, S, eps, gamma, beta, save_mean, save_invstd, g_scratch[dev],
                         kNoAllocScratchBytes, stream);
}
