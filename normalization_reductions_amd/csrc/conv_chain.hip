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
#include <stdlib.h>

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

// ---------------------------------------------------------------------------------------------
// Matrix-core producer: implicit GEMM on v_mfma_f32_16x16x4f32 (fp32 in, fp32 accumulate).
// Rows are output positions, columns output channels, K = (input channel, kd, kh, kw) padded
// to a multiple of 4 with zeros. Operand layouts of one instruction on gfx950 (checked on the
// device): A[m][k] comes from lane m + 16k, B[k][n] from lane n + 16k, and D[m][n] lands in lane
// n + 16*(m/4), register m%4. So lane l = r16 + 16q supplies A for position r16 and tap
// 4s + q, B for channel r16 and tap 4s + q, and receives channel r16 at 4 consecutive positions
// 4q..4q+3 -- one 16-byte store per (row tile, channel tile).
// Each lane keeps its weight fragment (KS x NT values) and its tap offsets into x in VGPRs for
// the whole wave; A is gathered from x (16 lanes read 16 consecutive positions of one tap).
// ---------------------------------------------------------------------------------------------
typedef float mf4 __attribute__((ext_vector_type(4)));
constexpr int kMfmaBlock = 256;  // 4 waves

template <int DIMS, int KS, int NT, int MT, int TPW>
__global__ __launch_bounds__(kMfmaBlock) void conv_k3_mfma_kernel(ConvGeom g, const float* __restrict__ x,
                                                                   const float* __restrict__ w,
                                                                   const float* __restrict__ b,
                                                                   float* __restrict__ c)
{
    constexpr int KD = DIMS == 3 ? 3 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int K = (int)g.Cin * KD * 9;
    const int plane = (int)(g.H * g.W);
    const int vol = (int)(g.D * plane);

    int koff[KS];
    float bw[KS][NT];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int k = 4 * s + q;
        const bool valid = k < K;
        const int ci = k / (KD * 9);
        const int rem = k - ci * (KD * 9);
        const int kd = rem / 9, kh = (rem % 9) / 3, kw = rem % 3;
        koff[s] = valid ? ci * vol + kd * plane + kh * (int)g.W + kw : 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bw[s][nt] = valid ? w[(int64_t)(nt * 16 + r16) * K + k] : 0.f;
    }
    float bias[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bias[nt] = b ? b[nt * 16 + r16] : 0.f;

    const int64_t n = blockIdx.y;
    const float* xn = x + n * g.Cin * (int64_t)vol;
    const int ohw = (int)(g.OH * g.OW);
    const bool vec_ok = (g.SP & 3) == 0;

    for (int t = 0; t < TPW; ++t) {
        const int64_t tile0 = (((int64_t)blockIdx.x * TPW + t) * (kMfmaBlock / 64) + wave) * (MT * 16);
        if (tile0 >= g.SP) break;
        int pbase[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t m = tile0 + mt * 16 + r16;
            int od = 0, oh = 0, ow = 0;
            if (m < g.SP) {
                const int mm = (int)m;
                od = DIMS == 3 ? mm / ohw : 0;
                const int r2 = mm - od * ohw;
                oh = r2 / (int)g.OW;
                ow = r2 - oh * (int)g.OW;
            }
            pbase[mt] = od * plane + oh * (int)g.W + ow;  // out-of-range rows read position 0
        }
        mf4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mf4{bias[nt], bias[nt], bias[nt], bias[nt]};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float av[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) av[mt] = xn[pbase[mt] + koff[s]];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mt], bw[s][nt], acc[mt][nt], 0, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t m0 = tile0 + mt * 16 + 4 * q;  // this lane's 4 positions
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float* dst = c + (n * g.Cout + nt * 16 + r16) * g.SP + m0;
                if (vec_ok && m0 + 3 < g.SP) {
                    *reinterpret_cast<mf4*>(dst) = acc[mt][nt];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (m0 + r < g.SP) dst[r] = acc[mt][nt][r];
                }
            }
        }
    }
}

// Eval-mode batch norm folded into the conv (BN page, its eval-mode discussion): per output
// channel k, a = gamma * scale / sqrt(rv + eps); W'[k][.] = W[k][.] * a and
// b' = ((b - rm) * gamma / sqrt(rv + eps) + beta) * scale. One workgroup per channel.
__global__ __launch_bounds__(256) void fold_bn_eval_kernel(const float* __restrict__ w,
                                                           const float* __restrict__ b,
                                                           const float* __restrict__ rm,
                                                           const float* __restrict__ rv,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ beta,
                                                           float eps, float scale, int64_t K,
                                                           float* __restrict__ wf, float* __restrict__ bf)
{
    const int64_t k = blockIdx.x;
    const float inv = 1.0f / sqrtf(rv[k] + eps);
    const float g = gamma ? gamma[k] : 1.f;
    const float a = g * inv * scale;
    for (int64_t j = threadIdx.x; j < K; j += 256) wf[k * K + j] = w[k * K + j] * a;
    if (threadIdx.x == 0) {
        const float bb = b ? b[k] : 0.f;
        const float bt = beta ? beta[k] : 0.f;
        bf[k] = ((bb - rm[k]) * g * inv + bt) * scale;
    }
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

// Four consecutive positions per thread (SP % 4 == 0, 16-byte aligned planes). The per-(n, k)
// coefficients are the same for the whole workgroup (n = blockIdx.y), so they come through
// scalar loads; each channel plane is read with coalesced 16-byte loads.
__global__ __launch_bounds__(kChainBlock) void chain_apply_vec_kernel(ChainArgs a)
{
    const int64_t i4 = (int64_t)blockIdx.x * kChainBlock + threadIdx.x;  // position / 4
    const int64_t n = blockIdx.y;
    if (4 * i4 >= a.SP) return;
    const f4* cp = reinterpret_cast<const f4*>(a.c + n * a.Cout * a.SP) + i4;
    const int64_t plane4 = a.SP / 4;
    f4 m = f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int64_t k = 0; k < a.Cout; ++k) {
        const GroupStat s = a.stats[a.batch ? k : n * a.Cout + k];
        const float pm = a.pre_mul ? a.pre_mul[k] : 1.f;
        const float A = s.rstd * (a.gamma ? a.gamma[k] : 1.f) * a.out_scale;
        const float B = (a.beta ? a.beta[k] : 0.f) * a.out_scale;
        const float qm = a.post_mul ? a.post_mul[k] : 1.f;
        const f4 cv = ld_stream(cp + k * plane4);
        f4 z = ((cv * pm - s.pivot) - s.mean_d) * A + B;
        if (a.clamp) {
            z.x = fminf(fmaxf(z.x, a.lo), a.hi);
            z.y = fminf(fmaxf(z.y, a.lo), a.hi);
            z.z = fminf(fmaxf(z.z, a.lo), a.hi);
            z.w = fminf(fmaxf(z.w, a.lo), a.hi);
        }
        z *= qm;
        if (a.reduce_max_c) {
            m.x = fmaxf(m.x, z.x);
            m.y = fmaxf(m.y, z.y);
            m.z = fmaxf(m.z, z.z);
            m.w = fmaxf(m.w, z.w);
        } else {
            st_stream(reinterpret_cast<f4*>(a.out + (n * a.Cout + k) * a.SP) + i4, z);
        }
    }
    if (a.reduce_max_c) st_stream(reinterpret_cast<f4*>(a.out + n * a.SP) + i4, m);
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

namespace {
template <int DIMS, int KS, int NT, int MT, int TPW>
hipError_t launch_mfma(const ConvGeom& g, const float* x, const float* w, const float* b, float* c,
                       hipStream_t stream)
{
    const int64_t per_wg = (int64_t)TPW * (kMfmaBlock / 64) * MT * 16;
    const dim3 grid((unsigned)((g.SP + per_wg - 1) / per_wg), (unsigned)g.N);
    conv_k3_mfma_kernel<DIMS, KS, NT, MT, TPW><<<grid, dim3(kMfmaBlock), 0, stream>>>(g, x, w, b, c);
    return hipGetLastError();
}

bool conv_valu_forced()
{
    const char* e = getenv("NORMRED_CONV");
    return e && e[0] == 'v';  // "valu": the vector-ALU producer (comparisons)
}
}  // namespace

hipError_t launch_conv_k3(const ConvGeom& g, const float* x, const float* w, const float* b,
                          float* c, hipStream_t stream)
{
    // Matrix-core producer for the compiled (dims, C_in, C_out) shapes; int32 offsets into one
    // batch item of x.
    const bool small = g.Cin * g.D * g.H * g.W < (1LL << 31) && g.SP < (1LL << 31);
    if (!conv_valu_forced() && small) {
        if (g.dims == 2 && g.Cin == 8 && g.Cout == 64)
            return launch_mfma<2, 18, 4, 4, 4>(g, x, w, b, c, stream);
        if (g.dims == 3 && g.Cin == 3 && g.Cout == 16)
            return launch_mfma<3, 21, 1, 8, 4>(g, x, w, b, c, stream);
    }
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
    const bool vec = (a.SP & 3) == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.c) | reinterpret_cast<uintptr_t>(a.out)) & 15) == 0;
    if (vec) {
        const int64_t n4 = a.SP / 4;
        const dim3 grid((unsigned)((n4 + kChainBlock - 1) / kChainBlock), (unsigned)a.N);
        chain_apply_vec_kernel<<<grid, dim3(kChainBlock), 0, stream>>>(a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((a.SP + kChainBlock - 1) / kChainBlock), (unsigned)a.N);
    chain_apply_kernel<<<grid, dim3(kChainBlock), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace nr

namespace nr {
hipError_t launch_fold_bn_eval(const ConvGeom& g, const float* w, const float* b, const float* rm,
                               const float* rv, const float* gamma, const float* beta, float eps,
                               float scale, float* wf, float* bf, hipStream_t stream)
{
    const int64_t K = g.Cin * (g.dims == 3 ? 27 : 9);
    fold_bn_eval_kernel<<<dim3((unsigned)g.Cout), dim3(256), 0, stream>>>(w, b, rm, rv, gamma, beta,
                                                                         eps, scale, K, wf, bf);
    return hipGetLastError();
}
}  // namespace nr
