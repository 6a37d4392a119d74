// Drives libnormred.so through its C ABI from plain C++: hipMalloc'd buffers, its own HIP
// stream, no Python or torch. It writes its input and the library's outputs as raw float32
// files into the directory given as argv[1]; the GPU test compares them with the oracle.
//
//   x.bin      x[3, 5, 100004], values from a counter-based generator (SplitMix64)
//   inorm.bin  inorm_forward(x)                      (read-once pipelined path)
//   noalloc.bin inorm_forward_noalloc(x)             (the same, in the library's own workspace)
//   bn.bin     bn_train_forward(x) * 2.0             (batch statistics per channel)
//   x5.bin, w5.bin, b5.bin, m5.bin, chain.bin
//              conv_norm_epilogue_forward on x5[2, 3, 6, 9, 11]: Conv3d 3 -> 16 (k = 3) ->
//              * m -> instance norm -> clamp [-1, 1] -> * m -> max over channels,
//              out [2, 4, 7, 9]
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
    std::vector<float> y(n), z(n), u(n);
    if (!hip_ok(hipMemcpy(y.data(), dy, n * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy y") ||
        !hip_ok(hipMemcpy(z.data(), dz, n * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy z"))
        return 1;
    // the entry point that allocates nothing, into z (bn's result is already on the host)
    if (!nr_ok(inorm_forward_noalloc(dx, dz, N, C, S, 1e-5f, nullptr, nullptr, nullptr, nullptr, st),
               "inorm_forward_noalloc") ||
        !hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize") ||
        !hip_ok(hipMemcpy(u.data(), dz, n * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy u"))
        return 1;

    // a small IN3d chain through the descriptor
    const int64_t cN = 2, cC = 3, cD = 6, cH = 9, cW = 11, cK = 16;
    std::vector<float> x5((size_t)(cN * cC * cD * cH * cW)), w5((size_t)(cK * cC * 27)), b5(cK), m5(cK);
    for (size_t i = 0; i < x5.size(); ++i)
        x5[i] = (float)((double)(splitmix64(0x5EED0300ull + i) >> 11) * 0x1.0p-53 * 4.0 - 2.0);
    for (size_t i = 0; i < w5.size(); ++i)
        w5[i] = (float)(((double)(splitmix64(0x5EED0400ull + i) >> 11) * 0x1.0p-53 - 0.5) * 0.4);
    for (int64_t k = 0; k < cK; ++k) {
        b5[k] = (float)(((double)(splitmix64(0x5EED0500ull + k) >> 11) * 0x1.0p-53 - 0.5));
        m5[k] = (float)(((double)(splitmix64(0x5EED0600ull + k) >> 11) * 0x1.0p-53 - 0.5) * 4.0);
    }
    const size_t nout = (size_t)(cN * (cD - 2) * (cH - 2) * (cW - 2));
    float *d5x = nullptr, *d5w = nullptr, *d5b = nullptr, *d5m = nullptr, *d5o = nullptr;
    void* ws5 = nullptr;
    nr_conv_norm_desc d{};
    d.spatial_dims = 3;
    d.ksize = 3;
    d.N = cN;
    d.C_in = cC;
    d.C_out = cK;
    d.in_d = cD;
    d.in_h = cH;
    d.in_w = cW;
    d.norm = NR_NORM_INSTANCE;
    d.eps = 1e-5f;
    d.out_scale = 1.0f;
    d.clamp = 1;
    d.clamp_lo = -1.0f;
    d.clamp_hi = 1.0f;
    d.reduce_max_c = 1;
    std::vector<float> out5(nout);
    if (!hip_ok(hipMalloc(&d5x, x5.size() * 4), "hipMalloc x5") ||
        !hip_ok(hipMalloc(&d5w, w5.size() * 4), "hipMalloc w5") ||
        !hip_ok(hipMalloc(&d5b, b5.size() * 4), "hipMalloc b5") ||
        !hip_ok(hipMalloc(&d5m, m5.size() * 4), "hipMalloc m5") ||
        !hip_ok(hipMalloc(&d5o, nout * 4), "hipMalloc out5") ||
        !hip_ok(hipMemcpy(d5x, x5.data(), x5.size() * 4, hipMemcpyHostToDevice), "hipMemcpy x5") ||
        !hip_ok(hipMemcpy(d5w, w5.data(), w5.size() * 4, hipMemcpyHostToDevice), "hipMemcpy w5") ||
        !hip_ok(hipMemcpy(d5b, b5.data(), b5.size() * 4, hipMemcpyHostToDevice), "hipMemcpy b5") ||
        !hip_ok(hipMemcpy(d5m, m5.data(), m5.size() * 4, hipMemcpyHostToDevice), "hipMemcpy m5"))
        return 1;
    d.pre_mul = d5m;
    d.post_mul = d5m;
    const size_t b5w = conv_norm_epilogue_workspace_size(&d);
    if (b5w == 0 || !hip_ok(hipMalloc(&ws5, b5w), "hipMalloc ws5") ||
        !nr_ok(conv_norm_epilogue_forward(&d, d5x, d5w, d5b, d5o, ws5, b5w, st),
               "conv_norm_epilogue_forward") ||
        !hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize") ||
        !hip_ok(hipMemcpy(out5.data(), d5o, nout * 4, hipMemcpyDeviceToHost), "hipMemcpy out5"))
        return 1;

    if (!write_file(dir + "/x.bin", x) || !write_file(dir + "/inorm.bin", y) ||
        !write_file(dir + "/bn.bin", z) || !write_file(dir + "/noalloc.bin", u) ||
        !write_file(dir + "/x5.bin", x5) || !write_file(dir + "/w5.bin", w5) ||
        !write_file(dir + "/b5.bin", b5) || !write_file(dir + "/m5.bin", m5) ||
        !write_file(dir + "/chain.bin", out5)) {
        std::fprintf(stderr, "cannot write the output files\n");
        return 1;
    }
    hipFree(d5x);
    hipFree(d5w);
    hipFree(d5b);
    hipFree(d5m);
    hipFree(d5o);
    hipFree(ws5);
    hipFree(dx);
    hipFree(dy);
    hipFree(dz);
    hipFree(ws1);
    hipFree(ws2);
    hipStreamDestroy(st);
    std::printf("ok\n");
    return 0;
}
