// conv_chain.hip -- k = 3 direct convolution producer and the normalize -> epilogue chain, gfx950.
//
// Conv: BN page (task l2_p73), its direct-conv kernel discussion: output (n, k, oh, ow) is the
// bias plus the sum over input channels and 3x3 taps of W[k, c, kh, kw] * x[n, c, oh+kh,
// ow+kw] (cross-correlation, valid, stride 1). IN3d page (task l2_p79): the 3-D form adds a
// depth tap; extents shrink by 2 along each axis.
//
// Mapping: one lane per output position, KB output channels per thread kept in registers.
// Every lane of a workgroup needs the same weight at the same time, so weights are read with
// wave-uniform addresses (scalar loads from the read-only weight buffer) and each loaded input
// value feeds KB fused multiply-adds. Inputs come through the vector L1/L2 path; neighbouring
// lanes share most of their taps.
//
// Chain: IN3d page, its step list and fused elementwise kernel (multiply, normalize, clamp,
// multiply, max over channels, each output position looping over the channels whose planes
// are read with coalesced accesses); BN page: normalize with batch statistics, affine, scale.
#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

constexpr int kConvBlock = 256;
constexpr int kKB = 16;  // output channels per thread

template <int DIMS, bool FULL>
__device__ __forceinline__ void conv_point(const ConvGeom& g, const float* __restrict__ x,
                                           const float* __restrict__ w,
                                           const float* __restrict__ b, float* __restrict__ c,
                                           int64_t n, int64_t k0, int64_t i)
{
    constexpr int KD = DIMS == 3 ? 3 : 1;
    int64_t od = 0, oh, ow;
    if (DIMS == 3) {
        const int64_t plane = g.OH * g.OW;
        od = i / plane;
        const int64_t r = i - od * plane;
        oh = r / g.OW;
        ow = r - oh * g.OW;
    } else {
        oh = i / g.OW;
        ow = i - oh * g.OW;
    }
    const int kcount = FULL ? kKB : (int)(g.Cout - k0);
    float acc[kKB];
#pragma unroll
    for (int k = 0; k < kKB; ++k) acc[k] = (k < kcount && b) ? b[k0 + k] : 0.f;

    for (int64_t ci = 0; ci < g.Cin; ++ci) {
        const float* xp = x + (((n * g.Cin + ci) * g.D + od) * g.H + oh) * g.W + ow;
        const float* wp = w + ((k0 * g.Cin + ci) * KD) * 9;
        const int64_t wk = g.Cin * KD * 9;  // stride between output channels in w
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) {
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) {
                    const float xv = xp[(kd * g.H + kh) * g.W + kw];
                    const int t = (kd * 3 + kh) * 3 + kw;
#pragma unroll
                    for (int k = 0; k < kKB; ++k)
                        if (k < kcount) acc[k] = fmaf(wp[k * wk + t], xv, acc[k]);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kKB; ++k)
        if (k < kcount) c[(n * g.Cout + k0 + k) * g.SP + i] = acc[k];
}

template <int DIMS>
__global__ __launch_bounds__(kConvBlock) void conv_k3_kernel(ConvGeom g, const float* __restrict__ x,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ b,
                                                              float* __restrict__ c)
{
    const int64_t i = (int64_t)blockIdx.x * kConvBlock + threadIdx.x;
    const int64_t n = blockIdx.y;
    const int64_t k0 = (int64_t)blockIdx.z * kKB;
    if (i >= g.SP) return;
    if (k0 + kKB <= g.Cout)
        conv_point<DIMS, true>(g, x, w, b, c, n, k0, i);
    else
        conv_point<DIMS, false>(g, x, w, b, c, n, k0, i);
}

constexpr int kChainBlock = 256;

__device__ __forceinline__ float chain_value(const ChainArgs& a, int64_t n, int64_t k, float cv)
{
    const GroupStat s = a.stats[a.batch ? k : n * a.Cout + k];
    const float pm = a.pre_mul ? a.pre_mul[k] : 1.f;
    const float A = s.rstd * (a.gamma ? a.gamma[k] : 1.f) * a.out_scale;
    const float B = (a.beta ? a.beta[k] : 0.f) * a.out_scale;
    float z = ((cv * pm - s.pivot) - s.mean_d) * A + B;
    if (a.clamp) z = fminf(fmaxf(z, a.lo), a.hi);
    if (a.post_mul) z *= a.post_mul[k];
    return z;
}

__global__ __launch_bounds__(kChainBlock) void chain_apply_kernel(ChainArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * kChainBlock + threadIdx.x;
    const int64_t n = blockIdx.y;
    if (i >= a.SP) return;
    if (a.reduce_max_c) {
        float m = -INFINITY;
        for (int64_t k = 0; k < a.Cout; ++k) {
            const float v = chain_value(a, n, k, ld_stream1(a.c + (n * a.Cout + k) * a.SP + i));
            m = fmaxf(m, v);
        }
        a.out[n * a.SP + i] = m;
    } else {
        for (int64_t k = 0; k < a.Cout; ++k) {
            const int64_t o = (n * a.Cout + k) * a.SP + i;
            a.out[o] = chain_value(a, n, k, ld_stream1(a.c + o));
        }
    }
}

}  // namespace

hipError_t launch_conv_k3(const ConvGeom& g, const float* x, const float* w, const float* b,
                          float* c, hipStream_t stream)
{
    const dim3 grid((unsigned)((g.SP + kConvBlock - 1) / kConvBlock), (unsigned)g.N,
                    (unsigned)((g.Cout + kKB - 1) / kKB));
    if (g.dims == 3)
        conv_k3_kernel<3><<<grid, dim3(kConvBlock), 0, stream>>>(g, x, w, b, c);
    else
        conv_k3_kernel<2><<<grid, dim3(kConvBlock), 0, stream>>>(g, x, w, b, c);
    return hipGetLastError();
}

hipError_t launch_chain_apply(const ChainArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.SP + kChainBlock - 1) / kChainBlock), (unsigned)a.N);
    chain_apply_kernel<<<grid, dim3(kChainBlock), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace nr
