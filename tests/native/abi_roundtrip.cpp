// Drives libnormred.so through its C ABI from plain C++: hipMalloc'd buffers, its own HIP
// stream, no Python or torch. It writes its input and the library's outputs as raw float32
// files into the directory given as argv[1]; the GPU test compares them with the oracle.
//
//   x.bin      x[3, 5, 100004], values from a counter-based generator (SplitMix64)
//   inorm.bin  inorm_forward(x)                      (read-once pipelined path)
//   bn.bin     bn_train_forward(x) * 2.0             (batch statistics per channel)
//
// Exit status 0 on success; a library error prints nr_last_error() and returns 1.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "normred.h"

namespace {

// SplitMix64 (Steele, Lea, Flood 2014): one 64-bit draw per element index.
uint64_t splitmix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

bool hip_ok(hipError_t e, const char* what)
{
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
}

bool nr_ok(nr_status s, const char* what)
{
    if (s == NR_OK) return true;
    std::fprintf(stderr, "%s failed (%d): %s\n", what, (int)s, nr_last_error());
    return false;
}

bool write_file(const std::string& path, const std::vector<float>& v)
{
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f) return false;
    const size_t n = std::fwrite(v.data(), sizeof(float), v.size(), f);
    std::fclose(f);
    return n == v.size();
}

}  // namespace

int main(int argc, char** argv)
{
    if (argc < 2) {
        std::fprintf(stderr, "usage: %s OUTPUT_DIR\n", argv[0]);
        return 2;
    }
    const std::string dir = argv[1];
    const int64_t N = 3, C = 5, S = 100004;
    const size_t n = (size_t)(N * C * S);
    std::vector<float> x(n);
    for (size_t i = 0; i < n; ++i) {
        const int64_t slice = (int64_t)(i / (size_t)S);
        const double u = (double)(splitmix64(0x5EED0200ull + i) >> 11) * 0x1.0p-53;  // [0, 1)
        x[i] = (float)((2.0 * u - 1.0) * (1.0 + 0.5 * (double)slice) + 0.25 * (double)(slice % 7));
    }

    std::printf("%s\n", nr_version());
    hipStream_t st;
    float *dx = nullptr, *dy = nullptr, *dz = nullptr;
    void *ws1 = nullptr, *ws2 = nullptr;
    const size_t b1 = inorm_workspace_size(N, C, S), b2 = bn_train_workspace_size(N, C, S);
    if (!hip_ok(hipStreamCreate(&st), "hipStreamCreate") ||
        !hip_ok(hipMalloc(&dx, n * sizeof(float)), "hipMalloc x") ||
        !hip_ok(hipMalloc(&dy, n * sizeof(float)), "hipMalloc y") ||
        !hip_ok(hipMalloc(&dz, n * sizeof(float)), "hipMalloc z") ||
        !hip_ok(hipMalloc(&ws1, b1), "hipMalloc ws1") || !hip_ok(hipMalloc(&ws2, b2), "hipMalloc ws2") ||
        !hip_ok(hipMemcpy(dx, x.data(), n * sizeof(float), hipMemcpyHostToDevice), "hipMemcpy x"))
        return 1;

    // a rejected call reports through the status and nr_last_error, before touching the GPU
    if (inorm_forward(nullptr, dy, N, C, S, 1e-5f, nullptr, nullptr, nullptr, nullptr, ws1, b1, st) !=
            NR_ERR_INVALID_ARG ||
        std::string(nr_last_error()).empty()) {
        std::fprintf(stderr, "a NULL input was not rejected\n");
        return 1;
    }

    if (!nr_ok(nr_workspace_clear(ws1, b1, st), "nr_workspace_clear") ||
        !nr_ok(nr_workspace_clear(ws2, b2, st), "nr_workspace_clear") ||
        !nr_ok(inorm_forward(dx, dy, N, C, S, 1e-5f, nullptr, nullptr, nullptr, nullptr, ws1, b1, st),
               "inorm_forward") ||
        !nr_ok(bn_train_forward(dx, dz, N, C, S, 1e-5f, nullptr, nullptr, 2.0f, nullptr, nullptr, ws2,
                                b2, st),
               "bn_train_forward"))
        return 1;
    uint32_t f1 = 0, f2 = 0;
    if (!nr_ok(nr_workspace_check(ws1, b1, st, &f1), "nr_workspace_check") ||
        !nr_ok(nr_workspace_check(ws2, b2, st, &f2), "nr_workspace_check"))
        return 1;
    if (f1 || f2) {
        std::fprintf(stderr, "workspace flags %u %u\n", f1, f2);
        return 1;
    }
    std::vector<float> y(n), z(n);
    if (!hip_ok(hipMemcpy(y.data(), dy, n * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy y") ||
        !hip_ok(hipMemcpy(z.data(), dz, n * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy z"))
        return 1;
    if (!write_file(dir + "/x.bin", x) || !write_file(dir + "/inorm.bin", y) ||
        !write_file(dir + "/bn.bin", z)) {
        std::fprintf(stderr, "cannot write the output files\n");
        return 1;
    }
    hipFree(dx);
    hipFree(dy);
    hipFree(dz);
    hipFree(ws1);
    hipFree(ws2);
    hipStreamDestroy(st);
    std::printf("ok\n");
    return 0;
}
