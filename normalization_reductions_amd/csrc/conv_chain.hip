// conv_chain.hip -- k = 3 direct convolution producer and the normalize -> epilogue chain, gfx950.
//
// Conv: BN page (task l2_p73), its direct-conv kernel discussion: output (n, k, oh, ow) is the
// bias plus the sum over input channels and 3x3 taps of W[k, c, kh, kw] * x[n, c, oh+kh,
// ow+kw] (cross-correlation, valid, stride 1). IN3d page (task l2_p79): the 3-D form adds a
// depth tap; extents shrink by 2 along each axis.
//
// Five producers, picked per shape by launch_conv_k3:
//   * conv2d_c8_bf16x6_kernel: 2-D, C_in 8 -> C_out 64, W 64 (the batch-norm model's shape) on
//     32x32x16 bf16 matrix instructions, each fp32 operand split exactly into three bf16 parts
//     and six of their products summed in fp32; workgroups own equal ranges of boxes of 4
//     output rows, staged in LDS, and store their tiles through a per-wave LDS transpose. Its
//     modes run the batch-norm chain by recomputation (a statistics pass storing nothing, then
//     the conv again with the normalize epilogue) and the eval chain (BN folded into W);
//   * conv2d_c8_mfma32_kernel: the same shape on 32x32x2 fp32 matrix instructions
//     (NORMRED_CONV=fp32);
//   * conv3d_c3_bf16x6_kernel: 3-D, C_in 3 -> C_out 16 over 32 x 32 input planes (the IN3d
//     model's shape) on 32x32x16 bf16 matrix instructions with the same exact splits, weights
//     as the A operand (16 channels x two weight parts), one output row per tile; persistent
//     workgroups roll a 3-slice LDS ring of split records over depth planes, and one LDS read
//     per tap row feeds its three kw taps through a wave-wide lane shift. It also takes the
//     instance statistics of its output, or folds eval-mode batch norm into W;
//   * conv_k3_ring_kernel: 2-D C_in 8 -> 64 of other widths and 3-D C_in 3 -> 16 of other
//     plane sizes on 16x16x4 fp32 matrix instructions, persistent workgroups rolling a 4-slice
//     LDS ring over rows or depth planes (NORMRED_CONV=fp32 takes it for 32 x 32 planes too);
//   * conv_k3_kernel: any other shape on the vector ALU, one lane per output position and KB
//     output channels per thread in registers; weights are read with wave-uniform addresses and
//     each loaded input value feeds KB fused multiply-adds.
//
// Chain: IN3d page, its step list and fused elementwise kernel (multiply, normalize, clamp,
// multiply, max over channels, each output position looping over the channels whose planes
// are read with coalesced accesses); BN page: normalize with batch statistics, affine, scale.
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

constexpr int kConvBlock = 256;
constexpr int kKB = 16;  // output channels per thread

template <int DIMS, bool FULL, bool CL>
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
        const float* xp = CL ? x + (((n * g.D + od) * g.H + oh) * g.W + ow) * g.Cin + ci
                             : x + (((n * g.Cin + ci) * g.D + od) * g.H + oh) * g.W + ow;
        const int64_t xs = CL ? g.Cin : 1;  // stride between neighbouring positions of x
        const float* wp = w + ((k0 * g.Cin + ci) * KD) * 9;
        const int64_t wk = g.Cin * KD * 9;  // stride between output channels in w
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) {
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) {
                    const float xv = xp[((kd * g.H + kh) * g.W + kw) * xs];
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
        if (k < kcount) {
            if (CL)
                c[(n * g.SP + i) * g.Cout + k0 + k] = acc[k];
            else
                c[(n * g.Cout + k0 + k) * g.SP + i] = acc[k];
        }
}

template <int DIMS, bool CL>
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
        conv_point<DIMS, true, CL>(g, x, w, b, c, n, k0, i);
    else
        conv_point<DIMS, false, CL>(g, x, w, b, c, n, k0, i);
}

// ---------------------------------------------------------------------------------------------
// Matrix-core producer: implicit GEMM on v_mfma_f32_16x16x4f32 (fp32 in, fp32 accumulate).
// Rows are output positions, columns output channels, K = (input channel, kd, kh, kw) padded
// to a multiple of 4 with zeros. Operand layouts of one instruction on gfx950 (checked on the
// device): A[m][k] comes from lane m + 16k, B[k][n] from lane n + 16k, and D[m][n] lands in lane
// n + 16*(m/4), register m%4. So lane l = r16 + 16q supplies A for position r16 and tap
// 4s + q, B for channel r16 and tap 4s + q, and receives channel r16 at 4 consecutive positions
// 4q..4q+3 -- one 16-byte store per (row tile, channel tile).
//
// Persistent form. The output is a sequence of outer slices (output rows in 2-D, output depth
// planes in 3-D), each cut into T tiles of 16 positions; the grid splits the N * OO * T tiles
// into equal contiguous ranges, one per workgroup. Output slice o of batch item n reads input
// slices o, o+1, o+2 of every input channel; a workgroup keeps those in a 4-slot LDS ring
// (slot = input slice mod 4, layout [slot][channel][slice]) and, while it computes slice o,
// loads input slice o+3 into registers and drops it into the free slot afterwards -- one new
// input slice per step, its latency hidden behind the step's matrix work. Each wave keeps the
// weights of one 16-channel tile for all K steps in VGPRs (B operands); A operands are LDS
// gathers (16 lanes read 16 consecutive positions of one tap).
//
// Tiles of a slice start `shift` positions early, shift = (o * positions per slice) mod 4, so
// every 4-position group a lane stores is 16-byte aligned in the output; positions outside the
// slice are computed from a dummy address and dropped.
// ---------------------------------------------------------------------------------------------
typedef float mf4 __attribute__((ext_vector_type(4)));
constexpr int kMfmaBlock = 256;  // 4 waves

// Floats of the ring producer's LDS before its statistics area: the larger of the 4-slot input
// ring and W plus the bias.
__host__ __device__ inline int ring_main_floats(const ConvGeom& g, const ConvRing& rg, int dims)
{
    const int ring_f = 4 * (int)g.Cin * rg.inner_in;
    const int w_f = (int)g.Cout * ((int)g.Cin * (dims == 3 ? 27 : 9) + 1);
    return ring_f > w_f ? ring_f : w_f;
}

// The workgroup holding tile t when `total` tiles are cut into G equal contiguous ranges
// [total * w / G, total * (w + 1) / G): the largest w with total * w / G <= t.
__host__ __device__ inline int64_t ring_wg_of(int64_t t, int64_t total, int64_t G)
{
    return ((t + 1) * G - 1) / total;
}

// Range index of workgroup b. Consecutive workgroup ids go round-robin over the 8 XCDs; ranges
// are given out so that each XCD's workgroups hold consecutive ranges (G a multiple of 8), so
// the input planes that neighbouring ranges share are read through the same L2.
__device__ __forceinline__ int64_t ring_range_of(int64_t b, int64_t G)
{
    return G % 8 == 0 ? (b % 8) * (G / 8) + b / 8 : b;
}

// Chan's merge of a step's statistics b (b.n > 0) into a lane's running statistics a, with the
// hardware reciprocal (1 ulp) for the weight: it runs once per tile step, inside the matrix
// loop. The exact merge (chan_merge) combines lanes, waves and workgroups. An empty a takes b
// as it is (the reciprocal's weight would round b's mean), and equal means merge exactly, so
// a constant channel keeps its value as the mean.
__device__ __forceinline__ Stat merge_step(Stat a, Stat b)
{
    Stat r;
    r.n = a.n + b.n;
    const float f = b.n * __builtin_amdgcn_rcpf(r.n);
    const float d = b.mean - a.mean;
    r.mean = fmaf(d, f, a.mean);
    r.m2 = a.m2 + b.m2 + d * d * a.n * f;
    return a.n > 0.f ? r : b;
}

// Two-pass statistics of V values (all valid), shifted by the first (the pivot) and summed as
// a tree: the mean is pivot + mean of the shifted values, exactly the value on a constant tile.
template <int V>
__device__ __forceinline__ Stat tile_stat(const float* v)
{
    const float K = v[0];
    float t[V];
#pragma unroll
    for (int i = 0; i < V; ++i) t[i] = v[i] - K;
#pragma unroll
    for (int w = 1; w < V; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < V; i += 2 * w) t[i] += t[i + w];
    const float md = t[0] * (1.f / V);
#pragma unroll
    for (int i = 0; i < V; ++i) t[i] = (v[i] - K - md) * (v[i] - K - md);
#pragma unroll
    for (int w = 1; w < V; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < V; i += 2 * w) t[i] += t[i + w];
    return Stat{(float)V, K + md, t[0]};
}

// Statistics of one tile step, from the lane's valid values. Planar: channel ch at positions
// p0 .. p0 + 3 of each of the MT tiles; channels last: channels 4q + r at position
// (t0 + mt) * 16 + r16. Steps whose tiles all lie inside the slice (the wave-uniform common
// case) skip the masks.
template <int MT, bool CL>
__device__ __forceinline__ void ring_tile_stats(const mf4* acc, int t0, int thi, int shift,
                                                int inner_out, int q, int r16, Stat* run, float* sh)
{
    const bool whole = t0 + MT <= thi && t0 * 16 - shift >= 0 && (t0 + MT) * 16 - shift <= inner_out;
    if (CL) {
        // channels last: MT values per channel and step, too few for a merge each; shifted sums
        // instead (run[r] holds the shift K in .mean, the sums of (v - K) and (v - K)^2 in .m2
        // and sh[r]), the shift being the lane's first value of the channel, so |mean - K|
        // stays within a few standard deviations, the final M2 = S2 - S1^2 / n loses little,
        // and a constant channel gives S1 = S2 = 0 and the value itself as the mean
        const bool first = run[0].n == 0.f;
        if (whole) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float K = first ? acc[0][r] : run[r].mean;
                float s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float d = acc[mt][r] - K;
                    s1 += d;
                    s2 = fmaf(d, d, s2);
                }
                run[r].mean = K;
                run[r].m2 += s2;
                run[r].n += (float)MT;
                sh[r] += s1;
            }
            return;
        }
        bool ok[MT];
        int cnt = 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            ok[mt] = t0 + mt < thi && (t0 + mt) * 16 + r16 < inner_out;
            cnt += ok[mt];
        }
        if (cnt == 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float first_v = 0.f;  // the lane's first valid value of channel 4q + r in this step
#pragma unroll
            for (int mt = MT - 1; mt >= 0; --mt) first_v = ok[mt] ? acc[mt][r] : first_v;
            const float K = first ? first_v : run[r].mean;
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float d = ok[mt] ? acc[mt][r] - K : 0.f;
                s1 += d;
                s2 = fmaf(d, d, s2);
            }
            run[r].mean = K;
            run[r].m2 += s2;
            run[r].n += (float)cnt;
            sh[r] += s1;
        }
        return;
    }
    // planar: 4 * MT values of channel ch per step, two-pass, merged into the running statistics
    if (whole) {
        float v[4 * MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) v[4 * mt + r] = acc[mt][r];
        run[0] = merge_step(run[0], tile_stat<4 * MT>(v));
        return;
    }
    bool ok[MT][4];
    int cnt = 0;
    float K = 0.f;  // pivot: the first valid value
#pragma unroll
    for (int mt = MT - 1; mt >= 0; --mt) {
        const int p0 = (t0 + mt) * 16 + 4 * q - shift;
#pragma unroll
        for (int r = 3; r >= 0; --r) {
            ok[mt][r] = t0 + mt < thi && p0 + r >= 0 && p0 + r < inner_out;
            cnt += ok[mt][r];
            K = ok[mt][r] ? acc[mt][r] : K;
        }
    }
    if (cnt == 0) return;
    float s = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s += ok[mt][r] ? acc[mt][r] - K : 0.f;
    const float md = s / (float)cnt;
    float m2 = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float d = ok[mt][r] ? acc[mt][r] - K - md : 0.f;
            m2 = fmaf(d, d, m2);
        }
    run[0] = merge_step(run[0], Stat{(float)cnt, K + md, m2});
}

__device__ __forceinline__ Stat shfl_xor_stat(Stat s, int off)
{
    return Stat{__shfl_xor(s.n, off), __shfl_xor(s.mean, off), __shfl_xor(s.m2, off)};
}

// End of this workgroup's part of batch item n: the lanes of a wave holding the same channel
// merge by a butterfly (lower lanes first), the waves of a channel tile in order of wm through
// LDS, and one thread per channel writes slot j = range - first_wg(n) of (n, k). Every
// thread of the workgroup calls it.
template <int WAVES_M, bool CL>
__device__ __forceinline__ void ring_stats_flush(const ConvGeom& g, const ConvRing& rg,
                                                 const RingStats& rs, float* lds, int64_t n,
                                                 int wm, int wn, int q, int r16, Stat* run)
{
    Stat* red = reinterpret_cast<Stat*>(lds);  // [WAVES_M][Cout]
    const int lane = threadIdx.x & 63;
    if (CL) {
        // lanes 16q .. 16q + 15 hold channels 4q .. 4q + 3 at 16 positions
#pragma unroll
        for (int off = 1; off < 16; off <<= 1)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const Stat o = shfl_xor_stat(run[r], off);
                run[r] = (lane & off) ? chan_merge(o, run[r]) : chan_merge(run[r], o);
            }
        if (r16 == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wm * (int)g.Cout + wn * 16 + 4 * q + r] = run[r];
        }
    } else {
        // lanes r16, r16 + 16, r16 + 32, r16 + 48 hold channel wn * 16 + r16
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            const Stat o = shfl_xor_stat(run[0], off);
            run[0] = (lane & off) ? chan_merge(o, run[0]) : chan_merge(run[0], o);
        }
        if (q == 0) red[wm * (int)g.Cout + wn * 16 + r16] = run[0];
    }
    __syncthreads();
    const int64_t tpn = (int64_t)rg.OO * rg.T;  // tiles per batch item
    const int64_t total = g.N * tpn;
    const int64_t first = ring_wg_of(n * tpn, total, gridDim.x);
    const int64_t wr = ring_range_of(blockIdx.x, gridDim.x);
    const int64_t j = wr - first;
    const bool last = ring_wg_of((n + 1) * tpn - 1, total, gridDim.x) == wr;
    for (int k = threadIdx.x; k < (int)g.Cout; k += kMfmaBlock) {
        Stat st = red[k];
        for (int m = 1; m < WAVES_M; ++m) st = chan_merge(st, red[m * (int)g.Cout + k]);
        const float pm = rs.pre_mul ? rs.pre_mul[k] : 1.f;
        float4* slot = rs.part + (n * rs.J) * g.Cout + k;
        slot[j * g.Cout] = make_float4(st.n, mul_rn(st.mean, pm), st.m2 * pm * pm, 0.f);
        if (last)
            for (int64_t jj = j + 1; jj < rs.J; ++jj) slot[jj * g.Cout] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
}

// With STATS the producer also takes the instance-norm statistics of its output while the
// tiles are in registers (IN3d page, its step list: statistics per (n, k) over the spatial
// extent; two-pass over each tile's values, merged by Chan's rule), so no pass re-reads c for
// them. Slot j of batch item n holds the part of n that workgroup first_wg(n) + j produced:
// (count, mean, M2, 0) of pre_mul * c per channel; the workgroup holding n's last tile marks
// the slots after its own empty, so a reader merges slots 0..J-1 of every item in order.
//
// The statistics cost registers: the variants taking them are held to 3 waves per SIMD (168
// VGPRs), and run at 3 workgroups per CU.
template <int DIMS, int KS, int WAVES_N, int MT, int PF, bool VEC, bool CL, bool STATS, bool P32 = false>
__global__ __launch_bounds__(kMfmaBlock) __attribute__((amdgpu_waves_per_eu(STATS ? 3 : 1, STATS ? 3 : 8)))
void conv_k3_ring_kernel(ConvGeom g, ConvRing rg,
                                                                   const float* __restrict__ x,
                                                                   const float* __restrict__ w,
                                                                   const float* __restrict__ b,
                                                                   float* __restrict__ c,
                                                                   RingStats rs, ConvFold fold)
{
    extern __shared__ float ring[];  // [4][Cin][inner_in], channels last: [4][inner_in][Cin]
    constexpr int KD = DIMS == 3 ? 3 : 1;
    constexpr int WAVES_M = (kMfmaBlock / 64) / WAVES_N;
    constexpr int NE = VEC ? PF : 4 * PF;  // elements (float4 or float) a thread moves per slice
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int Cin = (int)g.Cin;
    const int K = Cin * KD * 9;
    // P32: 3-D input planes of 32 x 32 (the IN3d model's), whose extents are then constants
    const int W = P32 ? 32 : (int)g.W;
    const int OW = P32 ? 30 : (int)g.OW;
    const int slice_floats = Cin * rg.inner_in;  // one input slice of every channel
    const int64_t cstride = (int64_t)rg.outer_in * rg.inner_in;

    // Element e of this thread is float (or float4) index i = e * 256 + tid of an input slice;
    // src[e] is its offset from the slice's start in x (-1: past the slice's end). Planar x
    // holds a slice as Cin runs of inner_in floats cstride apart; channels-last x holds it as
    // one contiguous run.
    int src[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int i = (e * kMfmaBlock + (int)threadIdx.x) * (VEC ? 4 : 1);
        const int ci = i / rg.inner_in;
        src[e] = i >= slice_floats ? -1 : CL ? i : (int)(ci * cstride) + (i - ci * rg.inner_in);
    }
    mf4 pf[PF];       // the next slice, loaded one step ahead
    mf4 rw[3][PF];    // the first run's window: its three slices, loaded together
    // Load input slice j of batch item n (all channels) into registers / store it into its slot.
    auto fetch = [&](mf4(&d)[PF], int64_t n, int j) {
        const float* xs = CL ? x + (n * rg.outer_in + j) * (int64_t)slice_floats
                             : x + n * Cin * cstride + (int64_t)j * rg.inner_in;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            if (src[e] < 0) continue;
            if (VEC)
                d[e] = *reinterpret_cast<const mf4*>(xs + src[e]);
            else
                d[e >> 2][e & 3] = xs[src[e]];
        }
    };
    auto drop = [&](const mf4(&d)[PF], int j) {
        float* dst = ring + (j & 3) * slice_floats + (int)threadIdx.x * (VEC ? 4 : 1);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            if (src[e] < 0) continue;
            if (VEC)
                *reinterpret_cast<mf4*>(dst + 4 * e * kMfmaBlock) = d[e];
            else
                dst[e * kMfmaBlock] = d[e >> 2][e & 3];
        }
    };
    const int64_t total = (int64_t)g.N * rg.OO * rg.T;
    const int64_t wr = ring_range_of(blockIdx.x, gridDim.x);
    const int64_t begin = total * wr / gridDim.x;
    const int64_t end = total * (wr + 1) / gridDim.x;

    // This lane's B fragment (channel ch, taps 4s + q): weight, outer tap a (kd in 3-D, kh in
    // 2-D) and the offset of the tap inside one slot, packed as (a << 24) | offset. W is read
    // once per workgroup with coalesced loads into the ring (free until the first window is
    // staged) and the lanes take their values from there: per-lane gathers would touch a cache
    // line per lane and load, and registers still awaiting a global load at the step loop make
    // the compiler wait for all loads in flight -- the next slice's prefetch included -- before
    // the tile loop.
    // The W loads are issued together, then the first run's window (its loads complete in order
    // behind W's, so the W staging waits for W alone); a loop that waited on each load in turn
    // and a window staged slice by slice put one memory latency per value or slice before the
    // first step.
    const int ch = wn * 16 + r16;
    const int wcount = (int)g.Cout * K;  // the launcher sizes the ring to hold W and the bias
    constexpr int WL = DIMS == 3 ? 6 : 18;  // W values per thread: 16 x 81 or 64 x 72
    float wv[WL];
#pragma unroll
    for (int k = 0; k < WL; ++k) {
        const int i = (int)threadIdx.x + k * kMfmaBlock;
        wv[k] = i < wcount ? w[i] : 0.f;
    }
    float bv = (int)threadIdx.x < (int)g.Cout && b ? b[threadIdx.x] : 0.f;
    if (fold.rv) {
        // eval mode folded in, with the fold kernel's arithmetic: channel factors once per
        // workgroup (C_out <= 64 for the ring's shapes), while the W loads are in flight
        __shared__ float fold_a[64];
        if ((int)threadIdx.x < (int)g.Cout) {
            const int k = threadIdx.x;
            const float inv = 1.0f / sqrtf(fold.rv[k] + fold.eps);
            const float gm = fold.gamma ? fold.gamma[k] : 1.f;
            fold_a[k] = gm * inv * fold.scale;
            const float bt = fold.beta ? fold.beta[k] : 0.f;
            bv = ((bv - fold.rm[k]) * gm * inv + bt) * fold.scale;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < WL; ++k) {
            const int i = (int)threadIdx.x + k * kMfmaBlock;
            if (i < wcount) wv[k] = wv[k] * fold_a[i / K];
        }
    }
    if (begin < end) {
        const int64_t sl = begin / rg.T, n = sl / rg.OO;
        const int o = (int)(sl - n * rg.OO);
#pragma unroll
        for (int j = 0; j < 3; ++j) fetch(rw[j], n, o + j);
    }
#pragma unroll
    for (int k = 0; k < WL; ++k) {
        const int i = (int)threadIdx.x + k * kMfmaBlock;
        if (i < wcount) ring[i] = wv[k];
    }
    for (int i = (int)threadIdx.x + WL * kMfmaBlock; i < wcount; i += kMfmaBlock) ring[i] = w[i];
    if ((int)threadIdx.x < (int)g.Cout) ring[wcount + threadIdx.x] = bv;
    for (int i = (int)threadIdx.x + kMfmaBlock; i < (int)g.Cout; i += kMfmaBlock) ring[wcount + i] = b ? b[i] : 0.f;
    __syncthreads();
    // The packed taps depend on q alone: a table [4][KS] in LDS after the ring (and the
    // statistics area), read once per slice, keeps them out of the step loop's registers.
    int* tapt = reinterpret_cast<int*>(ring + ring_main_floats(g, rg, DIMS) +
                                       (STATS ? WAVES_M * (int)g.Cout * 3 : 0));
    float bw[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int k = 4 * s + q;
        const bool valid = k < K;
        const int ci = k / (KD * 9);
        const int rem = k - ci * (KD * 9);
        int a, in_off;
        if (DIMS == 3) {
            a = rem / 9;
            in_off = ((rem % 9) / 3) * W + rem % 3;
        } else {
            a = rem / 3;
            in_off = rem % 3;
        }
        const int lds_off = CL ? in_off * Cin + ci : ci * rg.inner_in + in_off;
        if (wave == 0 && r16 == 0) tapt[q * KS + s] = valid ? (a << 24) | lds_off : 0;
        bw[s] = valid ? ring[ch * K + k] : 0.f;
    }
    // accumulator start: the bias of the channel(s) a lane's 4 results belong to (planar: its
    // channel ch at 4 positions; channels last: channels 4q..4q+3 of its tile at one position)
    mf4 bias4;
#pragma unroll
    for (int r = 0; r < 4; ++r) bias4[r] = ring[wcount + (CL ? wn * 16 + 4 * q + r : ch)];
    __syncthreads();
    // running statistics of this lane's channel(s) over the current batch item: planar, channel
    // ch; channels last, channels wn * 16 + 4q + r
    Stat run[CL ? 4 : 1];
    float sh[CL ? 4 : 1];  // channels last: sums of (v - shift), see ring_tile_stats
#pragma unroll
    for (int r = 0; r < (CL ? 4 : 1); ++r) {
        run[r] = stat_empty();
        sh[r] = 0.f;
    }

    if (begin < end) {  // the first run's window, loaded with W
        const int64_t sl = begin / rg.T, n = sl / rg.OO;
        const int o = (int)(sl - n * rg.OO);
#pragma unroll
        for (int j = 0; j < 3; ++j) drop(rw[j], o + j);
        __syncthreads();
    }
    int64_t cur = -1;  // global slice (n * OO + o) whose window is in the ring
    for (int64_t t = begin; t < end;) {
        const int64_t sl = t / rg.T;
        const int64_t n = sl / rg.OO;
        const int o = (int)(sl - n * rg.OO);
        const int tlo = (int)(t - sl * rg.T);
        const int thi = (int)min((int64_t)rg.T, end - sl * rg.T);
        if (cur >= 0 && (sl != cur + 1 || o == 0)) {  // a later run: stage its window slice by
            // slice (the registers of three slices would stay reserved in the loop)
#pragma unroll 1
            for (int j = o; j < o + 3; ++j) {
                fetch(pf, n, j);
                drop(pf, j);
            }
            __syncthreads();
        }
        const bool ahead = (sl + 1) * rg.T < end && o + 1 < rg.OO;  // next step continues this run
        if (ahead) fetch(pf, n, o + 3);

        // slot offsets of this step's taps
        int koff[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int tt = tapt[q * KS + s];
            koff[s] = ((o + (tt >> 24)) & 3) * slice_floats + (tt & 0xFFFFFF);
        }
        const int shift = (!CL && rg.vec_out) ? (int)(((int64_t)o * rg.inner_out) & 3) : 0;
        float* cs = c + (n * g.Cout + ch) * g.SP + (int64_t)o * rg.inner_out;

        // statistics of a step are taken one step late, between the next step's matrix
        // instructions, whose latency then covers them (the vector ALU issues while the matrix
        // unit runs); pt0 < 0: none pending
        mf4 pacc[MT];
        int pt0 = -1;
        for (int t0 = tlo + wm * MT; t0 < thi; t0 += WAVES_M * MT) {
            int base[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                int p = (t0 + mt) * 16 + r16 - shift;
                p = (p >= 0 && p < rg.inner_out && t0 + mt < thi) ? p : 0;
                if (DIMS == 3) {
                    const int oh = p / OW;
                    base[mt] = oh * W + (p - oh * OW);
                } else {
                    base[mt] = p;
                }
                if (CL) base[mt] *= Cin;
            }
            mf4 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = bias4;
            // channels last: D = W x X, so a lane receives 4 consecutive channels of one
            // position (D[m][n] lands in lane n + 16*(m/4), register m%4)
            auto mfma = [&](int s, int mt, float av) {
                acc[mt] = CL ? __builtin_amdgcn_mfma_f32_16x16x4f32(bw[s], av, acc[mt], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_16x16x4f32(av, bw[s], acc[mt], 0, 0, 0);
            };
            if (STATS) {
                // the gathers of 4 taps issued ahead of their matrix instructions: left to itself
                // the scheduler serializes each gather with its instruction in these variants
                constexpr int kB = 4;
#pragma unroll
                for (int s0 = 0; s0 < KS; s0 += kB) {
                    float av[kB][MT];
#pragma unroll
                    for (int i = 0; i < kB; ++i)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            if (s0 + i < KS) av[i][mt] = ring[base[mt] + koff[s0 + i]];
#pragma unroll
                    for (int i = 0; i < kB; ++i)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            if (s0 + i < KS) mfma(s0 + i, mt, av[i][mt]);
                    if (s0 == kB && pt0 >= 0)
                        ring_tile_stats<MT, CL>(pacc, pt0, thi, shift, rg.inner_out, q, r16, run, sh);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) pacc[mt] = acc[mt];
                pt0 = t0;
            } else {
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) mfma(s, mt, ring[base[mt] + koff[s]]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (t0 + mt >= thi) continue;
                if (CL) {
                    const int p = (t0 + mt) * 16 + r16;  // this lane's position
                    if (p >= rg.inner_out) continue;
                    float* dst = c + (n * g.SP + (int64_t)o * rg.inner_out + p) * g.Cout + wn * 16 + 4 * q;
                    if (rg.vec_out) {
                        *reinterpret_cast<mf4*>(dst) = acc[mt];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) dst[r] = acc[mt][r];
                    }
                    continue;
                }
                const int p0 = (t0 + mt) * 16 + 4 * q - shift;  // this lane's 4 positions
                if (rg.vec_out && p0 >= 0 && p0 + 3 < rg.inner_out) {
                    *reinterpret_cast<mf4*>(cs + p0) = acc[mt];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (p0 + r >= 0 && p0 + r < rg.inner_out) cs[p0 + r] = acc[mt][r];
                }
            }
        }
        if (STATS && pt0 >= 0)  // the slice's last step
            ring_tile_stats<MT, CL>(pacc, pt0, thi, shift, rg.inner_out, q, r16, run, sh);
        if (ahead) drop(pf, o + 3);
        __syncthreads();
        cur = sl;
        t = (sl + 1) * rg.T;
        if (STATS && (t >= end || o + 1 == rg.OO)) {  // this workgroup's part of item n is done
            if (CL) {
                // shifted sums to (count, mean, M2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float nn = run[r].n;
                    const float s1 = sh[r];
                    run[r] = nn > 0.f ? Stat{nn, run[r].mean + s1 / nn, fmaxf(run[r].m2 - s1 * s1 / nn, 0.f)}
                                      : stat_empty();
                }
            }
            ring_stats_flush<WAVES_M, CL>(g, rg, rs, ring + ring_main_floats(g, rg, DIMS), n, wm,
                                          wn, q, r16, run);
#pragma unroll
            for (int r = 0; r < (CL ? 4 : 1); ++r) {
                run[r] = stat_empty();
                sh[r] = 0.f;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// 2-D producer for C_in = 8, C_out = 64, W = 64 on v_mfma_f32_32x32x2f32 (the fp32 matrix
// instruction that keeps the pipe busiest on gfx950: ~150 TFLOP/s measured with register
// operands, against ~125-138 for 16x16x4). Lane l supplies A[m = l%32][k = l/32] (position m,
// tap 2s + l/32) and B[k][n = l%32] (channel, tap); D[m][n] lands in lane n + 32*((m/4)%2),
// register 4*(m/8) + m%4, so a lane stores channel l%32 at four aligned groups of 4 positions.
//
// A workgroup (4 waves) walks an equal contiguous range of boxes of B output rows of one batch
// item (the last box of an item may be shorter). A box's positions are cut into tiles of 32
// consecutive positions x all 64 channels, one tile per wave at a time; the two 32-channel
// accumulators of a tile share every A operand. The B + 2 input rows x 8 channels a box reads
// sit in LDS ([channel][row][64]), double-buffered: the next box's rows are loaded into
// registers while the current box's matrix work runs. With the row width fixed at compile time
// every tap's LDS offset is an immediate; a lane adds one of three per-tile bases (its
// position, plus the distance from its lane-half's first tap to its second: 1, W - 2 or
// B*W - 2).
// ---------------------------------------------------------------------------------------------
typedef float mf16 __attribute__((ext_vector_type(16)));
constexpr int kC8Cin = 8, kC8Cout = 64, kC8K = 72, kC8Steps = 36, kC8W = 64;

template <int B>
__global__ __launch_bounds__(256) void conv2d_c8_mfma32_kernel(ConvGeom g,
                                                               const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const float* __restrict__ b,
                                                               float* __restrict__ c)
{
    constexpr int W = kC8W, OW = W - 2;
    constexpr int ROWS = B + 2;                   // input rows a box reads
    constexpr int WIN = kC8Cin * ROWS * W;        // floats of one staged window
    constexpr int NE = (WIN / 4 + 255) / 256;     // float4 a thread stages per window
    constexpr int RUN4 = ROWS * W / 4;            // float4 per channel in a window
    __shared__ float win[2 * WIN];
    const int l = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = l & 31, kk = l >> 5;
    const int OH = (int)g.OH;
    const int64_t HW = g.H * W;
    const int nbox = (OH + B - 1) / B;

    // B operands: the workgroup reads W once with coalesced loads into LDS (the window buffers
    // are free until the first window is staged); each lane then takes its 72 values from there
    static_assert(kC8Cout * kC8K <= 2 * WIN, "W fits the window buffers");
    for (int i = (int)threadIdx.x; i < kC8Cout * kC8K; i += 256) win[i] = w[i];
    __syncthreads();
    float bw[2][kC8Steps];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int s = 0; s < kC8Steps; ++s) bw[nt][s] = win[(nt * 32 + m) * kC8K + 2 * s + kk];
    __syncthreads();
    const float bias0 = b ? b[m] : 0.f, bias1 = b ? b[32 + m] : 0.f;

    const int64_t total = g.N * (int64_t)nbox;
    const int64_t begin = total * blockIdx.x / gridDim.x;
    const int64_t end = total * (blockIdx.x + 1) / gridDim.x;
    mf4 pf[NE];
    // input rows o0 .. o0 + nout + 1 of every channel; rows past the box's need are not loaded
    auto fetch = [&](int64_t box) {
        const int64_t n = box / nbox;
        const int o0 = (int)(box - n * nbox) * B;
        const int run4 = (min(B, OH - o0) + 2) * (W / 4);
        const float* xs = x + n * kC8Cin * HW + (int64_t)o0 * W;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int i = e * 256 + (int)threadIdx.x;
            const int ci = i / RUN4;
            const int j = i - ci * RUN4;
            if (i < kC8Cin * RUN4 && j < run4)
                pf[e] = *reinterpret_cast<const mf4*>(xs + ci * HW + 4 * j);
        }
    };
    auto drop = [&](int buf) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int i = e * 256 + (int)threadIdx.x;
            if (i < kC8Cin * RUN4) *reinterpret_cast<mf4*>(win + buf * WIN + 4 * i) = pf[e];
        }
    };

    if (begin >= end) return;
    fetch(begin);
    drop(0);
    __syncthreads();
    int buf = 0;
    for (int64_t box = begin; box < end; ++box) {
        const bool more = box + 1 < end;
        if (more) fetch(box + 1);

        const int64_t n = box / nbox;
        const int o0 = (int)(box - n * nbox) * B;
        const int BP = min(B, OH - o0) * OW;  // positions in this box
        const int tiles = (BP + 31) / 32;
        float* c0 = c + (n * kC8Cout + m) * g.SP + (int64_t)o0 * OW;
        float* c1 = c0 + 32 * g.SP;
        for (int t = wave; t < tiles; t += 4) {
            int p = 32 * t + m;
            p = p < BP ? p : 0;
            const int r = p / OW;
            const float* a0 = win + buf * WIN + r * W + (p - r * OW);
            const float* a1 = a0 + kk;                // second tap: next column
            const float* a2 = a0 + kk * (W - 2);      // next row
            const float* a3 = a0 + kk * (B * W - 2);  // next channel
            mf16 acc0 = {}, acc1 = {};
#pragma unroll
            for (int s = 0; s < kC8Steps; ++s) {
                const int k0 = 2 * s;  // tap of lanes 0..31; lanes 32..63 take k0 + 1
                const int ci = k0 / 9, kh = (k0 % 9) / 3, kw = k0 % 3;
                const int off = ci * ROWS * W + kh * W + kw;
                const float av = kw < 2 ? a1[off] : kh < 2 ? a2[off] : a3[off];
                acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bw[0][s], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bw[1][s], acc1, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p0 = 32 * t + 8 * j + 4 * kk;  // positions of registers 4j..4j+3
                const mf4 v0 = mf4{acc0[4 * j], acc0[4 * j + 1], acc0[4 * j + 2], acc0[4 * j + 3]} + bias0;
                const mf4 v1 = mf4{acc1[4 * j], acc1[4 * j + 1], acc1[4 * j + 2], acc1[4 * j + 3]} + bias1;
                if (p0 + 3 < BP) {
                    *reinterpret_cast<mf4*>(c0 + p0) = v0;
                    *reinterpret_cast<mf4*>(c1 + p0) = v1;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (p0 + q < BP) {
                            c0[p0 + q] = v0[q];
                            c1[p0 + q] = v1[q];
                        }
                }
            }
        }
        if (more) drop(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
}

// ---------------------------------------------------------------------------------------------
// The same 2-D producer with its fp32 products formed on the bf16 matrix pipe. Every fp32
// value v splits exactly into three bf16 parts, v = h + m + l + e: h = RNE(v), m = RNE(v - h),
// l = RNE(v - h - m), where both differences are exact in fp32, and |e| <= 2^-24 |v|. A
// product x*w is taken as hh + hm + mh + mm + hl + lh. The dropped terms (ml, lm, ll) and the
// two remainders e are each at most 2^-24 |x w|, the size of one fp32 rounding, so the conv
// keeps fp32 accuracy. One v_mfma_f32_32x32x16_bf16 forms 16384 products in about half the
// time the fp32 32x32x2 instruction takes for 2048, so the six products' 27 instructions per 32
// channels (K = 72, below) need 2.7x fewer matrix cycles than fp32's 36.
//
// K order: a lane-half supplies one 3x3 tap with all 8 input channels, 8 bf16 that one 16-byte
// LDS read fetches, so the staged window is channels-last: [split][row][column][channel].
// Chunk q < 4 pairs tap 2q (lanes 0..31) with tap 2q + 1 (lanes 32..63), six instructions for
// its six products. Tap 8 fills the last chunk on its own: both lane halves take it, each with
// other parts ([xl | xm] x [wh | wm], [xm | xh] x [wh | wl], [xh | xh] x [wh | wm]), three
// instructions for the same six products -- 27 per 32 channels instead of the 30 a zero padding
// tap would take. A and B map (lane-half, element) to k the same way, so the products pair up
// in whatever order the instruction sums them. D has the 32x32 layout of the fp32 kernel above.
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef unsigned int mu4 __attribute__((ext_vector_type(4)));
typedef unsigned int mu2 __attribute__((ext_vector_type(2)));
constexpr int kBfChunks = 5;  // K = 72 -> 80: chunks of two taps x 8 channels

__device__ __forceinline__ unsigned bf16_rne(float v)
{
    const unsigned u = __float_as_uint(v);  // finite inputs: round to nearest even
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(unsigned h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ void split3(float v, unsigned& h, unsigned& m, unsigned& l)
{
    h = bf16_rne(v);
    const float r1 = v - bf16_value(h);
    m = bf16_rne(r1);
    l = bf16_rne(r1 - bf16_value(m));
}

// split3 of two values at once, each part packed as a pair (a in the low half): the hardware's
// packed conversion rounds to nearest even, so the parts are split3's, bit for bit
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float mf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split3x2(float a, float b, unsigned& h, unsigned& m, unsigned& l)
{
    h = __builtin_bit_cast(unsigned, __builtin_convertvector(mf2{a, b}, bf2));
    const float ra = a - __uint_as_float(h << 16), rb = b - __uint_as_float(h & 0xFFFF0000u);
    m = __builtin_bit_cast(unsigned, __builtin_convertvector(mf2{ra, rb}, bf2));
    const float la = ra - __uint_as_float(m << 16), lb = rb - __uint_as_float(m & 0xFFFF0000u);
    l = __builtin_bit_cast(unsigned, __builtin_convertvector(mf2{la, lb}, bf2));
}

constexpr uint32_t kC8Tag = 1u;  // the tag of a published word (cleared words carry 0)

// The apply pass's merge of channel ch: the statistics pass's nparts partials of the channel,
// thread-strided (thread t takes partials t, t + 256, ...), then a wave butterfly and the four
// waves in order -- a fixed order. Thread 0 publishes the mean and 1/sqrt(biased var + eps) as
// tagged words and blends the batch statistics into the running ones (BN page, opening
// analysis: running = (1 - m) * running + m * batch, with the unbiased batch variance). Every
// thread of the workgroup calls it; red holds 4 Stats of scratch.
__device__ __forceinline__ void c8_merge_publish(const C8Chain& e, const float* __restrict__ b, int ch, Stat* red)
{
    const float4* pp = e.part + (int64_t)ch * e.nparts;
    Stat st = lane_strided_merge<256>(e.nparts, [&](int64_t i) {
        const float4 p = pp[i];
        return Stat{p.x, p.y, p.z};
    });
    st = wave_merge<kWave>(st);
    if (lane_id() == 0) red[threadIdx.x / kWave] = st;
    __syncthreads();
    if (threadIdx.x == 0) {
        Stat t = red[0];
        for (int v = 1; v < 4; ++v) t = chan_merge(t, red[v]);
        const float rstd = rsqrtf(t.m2 / t.n + e.eps);
        xchg_store(e.xstats + 2 * ch, kC8Tag, t.mean);
        xchg_store(e.xstats + 2 * ch + 1, kC8Tag, rstd);
        if (e.run.mean) {
            // the statistics leave the bias out (see the statistics pass); the batch mean of
            // pre_mul * (conv + b) adds it back
            const float mo = e.run.momentum;
            const float bm = b ? mul_rn(b[ch], e.pre_mul ? e.pre_mul[ch] : 1.f) : 0.f;
            e.run.mean[ch] = (1.f - mo) * e.run.mean[ch] + mo * (t.mean + bm);
            e.run.var[ch] = (1.f - mo) * e.run.var[ch] + mo * (t.m2 / (t.n - 1.f));
        }
    }
    __syncthreads();
}

// Three modes share the producer: kC8Conv stores the conv output; kC8Stats stores nothing and
// writes each workgroup's per-channel (count, mean, M2) of the values conv * pre_mul, for
// batch-norm statistics; kC8Apply recomputes the conv and stores the normalized chain output
// ((v - mean) * rstd * gamma + beta) * out_scale, clamped, times post_mul, in the order the
// chain epilogue uses, with v = conv * pre_mul.
//
// The bias is left out of both: batch norm subtracts each channel's mean, so pre_mul * (conv +
// b) - mean(pre_mul * (conv + b)) is pre_mul * conv - mean(pre_mul * conv), and the apply pass
// saves an add per value (and the two roundings it brings). The running mean, which is not
// shift-invariant, adds pre_mul * b back.
//
// The statistics pass forms the same six products, in the same order, as the apply pass, so
// its statistics are those of the very values the apply pass normalizes. That matters on a
// channel of (near) zero variance, where any difference between the two passes' values is
// multiplied by 1/sqrt(eps): a constant input must give exactly beta * out_scale (BN page,
// opening training-mode analysis).
// kC8ApplyPlain is kC8Apply for chains without a pre-multiplier, clamp or post-multiplier (the
// batch-norm model's): it skips the multiplications by 1, which leave every value as it is.
enum { kC8Conv = 0, kC8Stats = 1, kC8Apply = 2, kC8ApplyPlain = 3 };

template <int B, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void conv2d_c8_bf16x6_kernel(ConvGeom g, const float* __restrict__ x, const float* __restrict__ w,
                             const float* __restrict__ b, float* __restrict__ c, C8Chain e)
{
    constexpr int W = kC8W, OW = W - 2;
    constexpr int NS = 3;                          // bf16 parts of each staged x value
    constexpr int ROWS = B + 2;                    // input rows a box reads
    constexpr int SPLIT = ROWS * W * kC8Cin;       // bf16 of one split of a staged window
    constexpr int WIN = NS * SPLIT;                // bf16 of one staged window
    constexpr int WSTAGE = 2 * kBfChunks * 3 * 64 * 8;  // bf16 of the staged B operands
    constexpr int ITEMS = ROWS * (W / 4) * 2;      // staging items: row x 4 columns x 4 channels
    static_assert(ITEMS <= 256, "one staging item per thread");
    constexpr int TPW = ((B * OW + 31) / 32 + 3) / 4;  // tiles of 32 positions per wave and box
    __shared__ __attribute__((aligned(16))) unsigned short win[2 * WIN > WSTAGE ? 2 * WIN : WSTAGE];
    // per-wave transpose of an output tile before its stores: 32 channels x 32 positions, rows
    // padded to 36 floats (144 bytes) so both the column writes and the row reads of 16 bytes
    // spread over the banks
    constexpr int TR = 36;
    __shared__ __attribute__((aligned(16))) float tr[MODE == kC8Stats ? 4 : 4 * 32 * TR];
    const int l = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = l & 31, kk = l >> 5;
    const int OH = (int)g.OH;
    const int64_t HW = g.H * W;
    const int nbox = (OH + B - 1) / B;

    const int64_t total = g.N * (int64_t)nbox;
    const int64_t wr = ring_range_of(blockIdx.x, gridDim.x);  // ranges by XCD (see there)
    const int64_t begin = total * wr / gridDim.x;
    const int64_t end = total * (wr + 1) / gridDim.x;
    // staging item of this thread: window row, 4 columns, 4 channels (consecutive threads take
    // consecutive columns, so each channel's loads are coalesced)
    const int it = threadIdx.x;
    const int srow = it >> 5, scq = (it >> 4) & 1, sj = it & 15;
    mf4 pf[4] = {};
    auto fetch = [&](int64_t box) {
        const int64_t n = box / nbox;
        const int o0 = (int)(box - n * nbox) * B;
        const int rows = min(B, OH - o0) + 2;  // rows past the box's need are not loaded
        if (it < ITEMS && srow < rows) {
            const float* xs = x + (n * kC8Cin + 4 * scq) * HW + (int64_t)(o0 + srow) * W + 4 * sj;
#pragma unroll
            for (int i = 0; i < 4; ++i) pf[i] = *reinterpret_cast<const mf4*>(xs + i * HW);
        }
    };

    // the statistics pass clears the words the apply pass publishes (stream order puts that
    // before the apply pass); the apply pass's first workgroups merge and publish them
    if (MODE == kC8Stats && blockIdx.x == 0)
        for (int i = (int)threadIdx.x; i < 2 * kC8Cout; i += 256)
            __hip_atomic_store(e.xstats + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    constexpr bool APPLY = MODE == kC8Apply || MODE == kC8ApplyPlain;
    if (APPLY)
        for (int ch = (int)blockIdx.x; ch < kC8Cout; ch += (int)gridDim.x)
            c8_merge_publish(e, b, ch, reinterpret_cast<Stat*>(win));

    // all of a thread's W loads are issued at once, then the first window's: the loads complete
    // in order, so the W staging waits for W alone while the window's loads are in flight
    constexpr int WPT = kC8Cout * kC8K / 256;
    static_assert(kC8Cout * kC8K % 256 == 0, "W values split evenly over the threads");
    // eval mode: the fold's per-channel parameters go out first, so the fold waits for them
    // alone (the loads complete in order)
    float f_rv = 1.f, f_gm = 1.f;
    if (MODE == kC8Conv && e.fold_rv && threadIdx.x < kC8Cout) {
        f_rv = e.fold_rv[threadIdx.x];
        if (e.gamma) f_gm = e.gamma[threadIdx.x];
    }
    float wv[WPT];
#pragma unroll
    for (int k = 0; k < WPT; ++k) wv[k] = w[(int)threadIdx.x + 256 * k];
    if (begin < end) fetch(begin);

    // B operands: lane l holds W[n][0..7][tap 2q + l/32] for n = 32 nt + l%32, in three splits.
    // The workgroup reads W once with coalesced loads, splits each value, and lays the splits
    // out in LDS as [nt][q][split][lane] x 8 bf16, from where every lane takes its operands
    // with 16-byte reads (gathering them per lane touched a cache line per lane and load).
    // The window buffers hold them until the first window is staged.
    // The last chunk holds tap 8 alone: both lane halves take it, each with other parts (see
    // the matrix loop), so its two operands are [h | m] and [h | l] of tap 8 (slots 0 and 1).
    static_assert(4 * kC8Cout * sizeof(Stat) <= 2 * WIN * sizeof(unsigned short), "partials fit");
    if (MODE == kC8Conv && e.fold_rv) {
        // eval mode folded in, with the fold kernel's arithmetic: each channel's factor once per
        // workgroup, while the W loads are in flight
        __shared__ float fold_a[kC8Cout];
        if (threadIdx.x < kC8Cout) fold_a[threadIdx.x] = f_gm * (1.0f / sqrtf(f_rv + e.eps)) * e.out_scale;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < WPT; ++k) wv[k] = wv[k] * fold_a[((int)threadIdx.x + 256 * k) / kC8K];
    }
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
        const int i = (int)threadIdx.x + 256 * k;
        const int n = i / kC8K, rem = i - n * kC8K, ci = rem / 9, tap = rem - ci * 9;
        unsigned h, mm, lo;
        split3(wv[k], h, mm, lo);
        unsigned short* d = win + (((n >> 5) * kBfChunks + (tap >> 1)) * 3 * 64 + (n & 31) + 32 * (tap & 1)) * 8 + ci;
        if (tap < 8) {
            d[0] = (unsigned short)h;
            d[64 * 8] = (unsigned short)mm;
            d[2 * 64 * 8] = (unsigned short)lo;
        } else {
            d[0] = d[64 * 8] = (unsigned short)h;      // lanes 0..31 of slots 0, 1: h
            d[32 * 8] = (unsigned short)mm;            // lanes 32..63: m (slot 0), l (slot 1)
            d[(64 + 32) * 8] = (unsigned short)lo;
        }
    }
    __syncthreads();
    bf8 wb[2][kBfChunks][3];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int q = 0; q < kBfChunks; ++q)
#pragma unroll
            for (int sp = 0; sp < (q < kBfChunks - 1 ? 3 : 2); ++sp)
                wb[nt][q][sp] = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(win + (((nt * kBfChunks + q) * 3 + sp) * 64 + l) * 8));
    __syncthreads();
    float bias0 = b ? b[m] : 0.f, bias1 = b ? b[32 + m] : 0.f;
    if (MODE == kC8Conv && e.fold_rv) {
        auto fold_b = [&](int k, float bb) {
            const float inv = 1.0f / sqrtf(e.fold_rv[k] + e.eps);
            const float gm = e.gamma ? e.gamma[k] : 1.f;
            const float bt = e.beta ? e.beta[k] : 0.f;
            return ((bb - e.fold_rm[k]) * gm * inv + bt) * e.out_scale;
        };
        bias0 = fold_b(m, bias0);
        bias1 = fold_b(32 + m, bias1);
    }
    // per-channel factors of this lane's two channels m and 32 + m
    float pm0 = 1.f, pm1 = 1.f, mu0 = 0.f, mu1 = 0.f, A0 = 1.f, A1 = 1.f, B0 = 0.f, B1 = 0.f, q0 = 1.f, q1 = 1.f;
    if (MODE != kC8Conv && e.pre_mul) {
        pm0 = e.pre_mul[m];
        pm1 = e.pre_mul[32 + m];
    }
    if (APPLY) {
        A0 = (e.gamma ? e.gamma[m] : 1.f) * e.out_scale;  // times rstd once it is published
        A1 = (e.gamma ? e.gamma[32 + m] : 1.f) * e.out_scale;
        B0 = (e.beta ? e.beta[m] : 0.f) * e.out_scale;
        B1 = (e.beta ? e.beta[32 + m] : 0.f) * e.out_scale;
        if (e.post_mul) {
            q0 = e.post_mul[m];
            q1 = e.post_mul[32 + m];
        }
    }
    // The channel statistics, read before the first epilogue (after the first tile's matrix
    // work, which hides the merge): a bounded wait for the four tagged words of channels m and
    // 32 + m; if it gives up it raises the sticky flag (the results are then invalid).
    bool have_stats = !APPLY;
    auto fetch_stats = [&]() {
        unsigned long long w0, w1, w2, w3;
        uint32_t spins = 0;
        for (;;) {
            w0 = xchg_load(e.xstats + 2 * m);
            w1 = xchg_load(e.xstats + 2 * m + 1);
            w2 = xchg_load(e.xstats + 2 * (32 + m));
            w3 = xchg_load(e.xstats + 2 * (32 + m) + 1);
            if ((uint32_t)(w0 >> 32) == e.wait_tag && (uint32_t)(w1 >> 32) == e.wait_tag &&
                (uint32_t)(w2 >> 32) == e.wait_tag && (uint32_t)(w3 >> 32) == e.wait_tag)
                break;
            if (++spins > e.spin_limit) {
                raise_flag(e.flags, kFlagSpinTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        mu0 = __uint_as_float((uint32_t)w0);
        A0 *= __uint_as_float((uint32_t)w1);
        mu1 = __uint_as_float((uint32_t)w2);
        A1 *= __uint_as_float((uint32_t)w3);
        have_stats = true;
    };
    float K0 = 0.f, K1 = 0.f, cnt = 0.f, sum0 = 0.f, sum1 = 0.f, sq0 = 0.f, sq1 = 0.f;

    auto drop = [&](int buf) {
        if (it < ITEMS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                unsigned h01, m01, l01, h23, m23, l23;
                split3x2(pf[0][e], pf[1][e], h01, m01, l01);
                split3x2(pf[2][e], pf[3][e], h23, m23, l23);
                unsigned short* d = win + buf * WIN + (srow * W + 4 * sj + e) * kC8Cin + 4 * scq;
                *reinterpret_cast<mu2*>(d) = mu2{h01, h23};
                *reinterpret_cast<mu2*>(d + SPLIT) = mu2{m01, m23};
                *reinterpret_cast<mu2*>(d + 2 * SPLIT) = mu2{l01, l23};
            }
        }
    };

    if (begin >= end) {  // (the grid never exceeds the boxes; an empty partial all the same)
        if (MODE == kC8Stats && threadIdx.x < kC8Cout)
            e.part[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = float4{0.f, 0.f, 0.f, 0.f};
        return;
    }
    drop(0);
    __syncthreads();
    int buf = 0;
    for (int64_t box = begin; box < end; ++box) {
        const bool more = box + 1 < end;
        if (more) fetch(box + 1);

        const int64_t n = box / nbox;
        const int o0 = (int)(box - n * nbox) * B;
        const int BP = min(B, OH - o0) * OW;  // positions in this box: a multiple of 4, >= 62
        // lane l stores 16 bytes of channel l / 8 + 8 s at position 4 (l % 8) of a tile
        // stores through a buffer resource over batch item n's output (64 SP floats, below 2^31
        // bytes): the lane's byte offset in a register, channel block (32 h + 8 s)'s in a scalar
        // register, so no store needs its own 64-bit address arithmetic
        const __amdgpu_buffer_rsrc_t cres = __builtin_amdgcn_make_buffer_rsrc(
            MODE == kC8Stats ? (float*)nullptr : c + n * kC8Cout * g.SP, 0, (int)(kC8Cout * g.SP * 4),
            0x00020000 /* 32-bit data format */);
        const int lane_off = (int)(((l >> 3) * g.SP + o0 * OW + 4 * (l & 7)) * 4);
        // exactly TPW tiles per wave, each 32 whole positions of the box: the last tile ends at
        // the box's last position (overlapping the one before), and waves with no tile left
        // repeat the last. Overlaps rewrite bitwise-identical values, and every lane issues the
        // same 8 TPW stores per box, so the wait for the next box's loads need not wait for them.
        const int tiles = (BP + 31) / 32;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int ts = min(32 * min(wave + 4 * i, tiles - 1), BP - 32);
            const int p = ts + m;
            const int r = p / OW;
            // window position of this lane's tap (0, 0), then the lane-half distances: one
            // column (chunks 0, 2, 3: taps 0|1, 4|5, 6|7), W - 2 (chunk 1: taps 2|3), none
            // (chunk 4: tap 8 | padding)
            const unsigned short* a0 = win + buf * WIN + (r * W + (p - r * OW)) * kC8Cin;
            const unsigned short* a1 = a0 + kk * kC8Cin;
            const unsigned short* a2 = a0 + kk * (W - 2) * kC8Cin;
            mf16 acc0 = {}, acc1 = {};
            // the statistics pass gains from the scheduler's interleave of LDS reads and matrix
            // instructions (-6 %); the storing passes do not
            if (MODE == kC8Stats) __builtin_amdgcn_iglp_opt(1);
#pragma unroll
            for (int q = 0; q < kBfChunks - 1; ++q) {
                const int off = (q == 0 ? 0 : q == 1 ? 2 : q == 2 ? W + 1 : 2 * W) * kC8Cin;
                const unsigned short* a = q == 1 ? a2 : a1;
                const bf8 ah = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(a + off));
                const bf8 am = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(a + off + SPLIT));
                const bf8 al = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(a + off + 2 * SPLIT));
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, wb[0][q][1], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, wb[1][q][1], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, wb[0][q][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, wb[1][q][0], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wb[0][q][2], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wb[1][q][2], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wb[0][q][1], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wb[1][q][1], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, wb[0][q][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, wb[1][q][0], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wb[0][q][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wb[1][q][0], acc1, 0, 0, 0);
            }
            {
                // tap 8 in both lane halves, three instructions for its six products (smallest
                // first): [xl | xm] x [wh | wm] = lh, mm; [xm | xh] x [wh | wl] = mh, hl;
                // [xh | xh] x [wh | wm] = hh, hm. Half 1 reads the next part down of half 0's.
                const unsigned short* a = a0 + (2 * W + 2) * kC8Cin + (kk ? 0 : SPLIT);
                const bf8 xh = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(a0 + (2 * W + 2) * kC8Cin));
                const bf8 xb = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(a));
                const bf8 xc = __builtin_bit_cast(bf8, *reinterpret_cast<const mu4*>(a + SPLIT));
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xc, wb[0][kBfChunks - 1][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xc, wb[1][kBfChunks - 1][0], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb, wb[0][kBfChunks - 1][1], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb, wb[1][kBfChunks - 1][1], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, wb[0][kBfChunks - 1][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, wb[1][kBfChunks - 1][0], acc1, 0, 0, 0);
            }
            if (MODE == kC8Stats) {
                // positions this tile owns: from 32 t on for a tile t < tiles (an overlapping
                // last tile starts earlier), none for a repeated tile. A lane's registers hold
                // positions ts + 8 (r / 4) + 4 kk + r % 4, increasing with r, so it owns the
                // registers from r0 on. Each lane sums the raw conv sums shifted by its pivot
                // (its first value of a tile with owned values, so a constant channel sums exact
                // zeros and keeps the pivot as its mean): per tile, then into the lane's totals. The
                // pre-multiplier enters once per workgroup (mean m * pm, M2 * pm^2) when the partial is
                // written, rounded as the apply pass rounds each value.
                const int t = wave + 4 * i;
                const int own = t < tiles ? 32 * t : BP;
                if (cnt == 0.f) {  // nothing summed yet: (re)take the pivot
                    K0 = acc0[0];
                    K1 = acc1[0];
                }
                acc0 -= K0;
                acc1 -= K1;
                if (ts < own) {  // a box's overlapping last tile or a repeated tile
                    // not-owned registers: 4 for each whole 8 positions before own, then the
                    // rest of that group of 4
                    const int lead = max(0, own - ts - 4 * kk);
                    const int r0 = min(16, 4 * (lead >> 3) + min(4, lead & 7));
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc0[r] = r >= r0 ? acc0[r] : 0.f;
                        acc1[r] = r >= r0 ? acc1[r] : 0.f;
                    }
                    cnt += (float)(16 - r0);
                } else {
                    cnt += 16.f;
                }
                float s0 = 0.f, s1 = 0.f, d0 = 0.f, d1 = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s0 += acc0[r];
                    s1 += acc1[r];
                    d0 = fmaf(acc0[r], acc0[r], d0);
                    d1 = fmaf(acc1[r], acc1[r], d1);
                }
                sum0 += s0;
                sum1 += s1;
                sq0 += d0;
                sq1 += d1;
            } else {
                if (!have_stats) fetch_stats();
                // the lane's values are channel m (acc0) or 32 + m (acc1) at positions
                // ts + 8 j + 4 kk + 0..3; the epilogue runs on them as they are, then the wave
                // transposes each 32 x 32 tile through its LDS rows so that 8 consecutive lanes
                // store 128 contiguous bytes of one channel
                float* trw = tr + wave * 32 * TR;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const mf16& acc = h ? acc1 : acc0;
                    const float bias = h ? bias1 : bias0, pm = h ? pm1 : pm0, mu = h ? mu1 : mu0;
                    const float A = h ? A1 : A0, Bc = h ? B1 : B0, qm = h ? q1 : q0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        mf4 z = mf4{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
                        if (MODE == kC8Conv) z += bias;  // batch norm: the bias cancels (see above)
                        if (MODE == kC8ApplyPlain) {
                            z = (z - mu) * A + Bc;
                        } else if (MODE == kC8Apply) {
                            z = (mul_rn(z, pm) - mu) * A + Bc;
                            if (e.clamp) {
#pragma unroll
                                for (int r = 0; r < 4; ++r) z[r] = fminf(fmaxf(z[r], e.lo), e.hi);
                            }
                            z *= qm;
                        }
                        *reinterpret_cast<mf4*>(trw + m * TR + 8 * j + 4 * kk) = z;
                    }
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const mf4 z = *reinterpret_cast<const mf4*>(trw + ((l >> 3) + 8 * s) * TR + 4 * (l & 7));
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(mu4, z), cres, lane_off + 4 * ts,
                                                               (int)((32 * h + 8 * s) * g.SP * 4), 0);
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
        if (more) drop(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    if (MODE == kC8Stats) {
        // the lane's statistics from its shifted sums, then the lane halves (they hold the same
        // channels; lower half first), then the waves in order
        Stat run0 = stat_empty(), run1 = stat_empty();
        if (cnt > 0.f) {
            const float rn = __builtin_amdgcn_rcpf(cnt), md0 = sum0 * rn, md1 = sum1 * rn;
            const float v0 = sq0 - sum0 * md0, v1 = sq1 - sum1 * md1;  // >= 0 but for rounding
            run0 = Stat{cnt, K0 + md0, v0 < 0.f ? 0.f : v0};
            run1 = Stat{cnt, K1 + md1, v1 < 0.f ? 0.f : v1};
        }
        Stat o0, o1;
        o0.n = __shfl_xor(run0.n, 32);
        o0.mean = __shfl_xor(run0.mean, 32);
        o0.m2 = __shfl_xor(run0.m2, 32);
        o1.n = __shfl_xor(run1.n, 32);
        o1.mean = __shfl_xor(run1.mean, 32);
        o1.m2 = __shfl_xor(run1.m2, 32);
        run0 = kk ? chan_merge(o0, run0) : chan_merge(run0, o0);
        run1 = kk ? chan_merge(o1, run1) : chan_merge(run1, o1);
        Stat* red = reinterpret_cast<Stat*>(win);  // [wave][channel]; the windows are done
        if (kk == 0) {
            red[wave * kC8Cout + m] = run0;
            red[wave * kC8Cout + 32 + m] = run1;
        }
        __syncthreads();
        if (threadIdx.x < kC8Cout) {
            const int ch = threadIdx.x;
            Stat t = red[ch];
#pragma unroll
            for (int v = 1; v < 4; ++v) t = chan_merge(t, red[v * kC8Cout + ch]);
            const float pc = e.pre_mul ? e.pre_mul[ch] : 1.f;
            e.part[(int64_t)ch * gridDim.x + blockIdx.x] = float4{t.n, mul_rn(t.mean, pc), t.m2 * pc * pc, 0.f};
        }
    }
}

// ---------------------------------------------------------------------------------------------
// 3-D producer for C_in = 3 -> C_out = 16 over 32 x 32 input planes (the IN3d model's shape),
// its fp32 products formed on the bf16 matrix pipe from the exact three-part splits of the 2-D
// producer above. The operand roles are swapped against that producer: A holds the weights and
// B the input, so one v_mfma_f32_32x32x16_bf16 covers 32 output positions (its columns) x 32
// rows, and the rows hold the 16 output channels twice, rows 0..15 with one weight part and
// rows 16..31 with another. A tap contributes 12 K elements, its three channels' splits
// (xh, xm, xl, xh), weighted (Wh, Wh, Wh, Wl) in the upper rows and (Wm, Wm, Wm, 0) in the lower
// ones: the upper rows sum hh + hm + hl + lh, the lower ones mh + mm + ml, and the two halves
// added hold the six products of the 2-D producer plus ml (which only adds accuracy). With 16
// output channels the fp32 instruction (16x16x4) needs 21 steps of 32 cycles per 16 positions;
// this needs 21 of 32 cycles per 32 positions (28 taps x 12 / 16), 2x fewer matrix cycles.
//
// K order: each lane half walks its own sequence of 14 taps (below), 12 elements a tap, 8
// elements an instruction, so two taps fill three instructions. A staged record -- one input
// position, 24 bytes -- holds a tap's 12 elements as three 8-byte pieces in three areas of the
// slot ([h0 h1 h2 m0], [m1 m2 l0 l1], [l2 h0 h1 h2]), each one LDS read. A and B map (lane
// half, element) to (tap, channel, part) alike. D: lane l receives position l % 32, rows
// 8j + 4(l / 32) + r in register 4j + r, so after adding the row halves it holds output
// channels 4(l / 32) + r and 8 + 4(l / 32) + r (r = 0..3) of one position.
//
// Persistent form as the fp32 ring producer: a tile is one output row (30 positions; lanes 30
// and 31 repeat lane 29's reads and store nothing), each output depth slice holds 30 of them,
// and the grid splits the N * OD * 30 tiles into equal contiguous ranges, given out by XCD.
// Row tiles cost no more matrix rounds than tiles of 32 consecutive positions would (29 per
// slice: 4 rounds of 8 either way), and their reads are free of LDS bank conflicts: 32
// consecutive positions cross a row, and the two lanes past the row's end hit the banks of the
// row's first two records. The window of output slice o -- input slices o, o+1, o+2 -- sits in
// LDS as those 24-byte records: a ring of three 24 KB slots, so two workgroups share a CU. The
// next input slice is loaded into registers during a step, then split and packed into slice o's
// slot once every wave is done with it.
// ---------------------------------------------------------------------------------------------
constexpr int k3Pos = 900, k3Tiles = 30;  // positions and row tiles per output depth slice
// ushorts of one area (an 8-byte piece of every position's record) of a staged input slice,
// padded by 16 bytes: areas 8208 bytes apart are read with one instruction each, straight into
// the operand's registers (at 8192 the compiler pairs two areas of a tap into one read and then
// shuffles registers); the padding keeps the staging's 16-byte writes aligned
constexpr int k3SplitU = 1024 * 4 + 8;
constexpr int k3SlotU = 3 * k3SplitU;
constexpr int k3Ops = 21;  // matrix instructions per tile: 14 taps x 12 elements / 8
constexpr int k3Wgs = 2;   // workgroups per CU (the LDS holds two rings)

// Tap sequence of a lane half. A tap row is (kd, kh), R = 3 kd + kh, holding taps 3R + kw. Half
// 0 takes rows 0..3 and half 1 rows 4..7, each as kw = 0, 1, 2, so the halves run the same kw
// sequence; row 8 comes last, kw 0, 1 in half 0 and kw 2 and the padding tap (27, zero weight)
// in half 1. Tap j (0..13) of half kk:
__device__ __forceinline__ int k3_tap(int kk, int j)
{
    if (j < 12) return 3 * (4 * kk + j / 3) + j % 3;
    return j == 12 ? (kk ? 26 : 24) : (kk ? 27 : 25);
}

// Lane l takes lane l + 1's value (a wave-wide shift; the last lane gets 0): tap kw + 1 of
// output column c is tap kw of column c + 1, so one LDS read per tap row feeds all three kw.
__device__ __forceinline__ unsigned k3_next_lane(unsigned v)
{
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x130 /* wave_shl:1 */, 0xF, 0xF, true);
}

template <bool CL, bool STATS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void conv3d_c3_bf16x6_kernel(ConvGeom g, const float* __restrict__ x, const float* __restrict__ w,
                             const float* __restrict__ b, float* __restrict__ c, RingStats rs,
                             ConvFold fold)
{
    __shared__ __attribute__((aligned(16))) unsigned short ring3[3 * k3SlotU];
    __shared__ float bias3[16];
    __shared__ Stat red3[4 * 16];
    const int tid = threadIdx.x;
    const int l = tid & 63, wave = tid >> 6;
    const int m = l & 31, kk = l >> 5;
    const int D = (int)g.D, OD = (int)g.OD;
    const int64_t SP = g.SP;
    const int64_t total = g.N * (int64_t)OD * k3Tiles;
    const int64_t G = gridDim.x;
    const int64_t wr = ring_range_of(blockIdx.x, G);
    const int64_t begin = total * wr / G;
    const int64_t end = total * (wr + 1) / G;

    // staging: thread t moves positions 4t .. 4t + 3 of an input slice, its three channels
    auto fetch = [&](mf4(&f)[3], int64_t n, int z) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            f[k] = CL ? *reinterpret_cast<const mf4*>(x + ((n * D + z) * 1024) * 3 + 12 * tid + 4 * k)
                      : *reinterpret_cast<const mf4*>(x + ((n * 3 + k) * D + z) * 1024 + 4 * tid);
    };
    auto drop = [&](const mf4(&f)[3], int z) {
        // the records of the thread's 4 positions: area a in r[8 a .. 8 a + 7], position j's
        // 8 bytes at 2j, 2j + 1 (bf16 pairs, the first element in the low half)
        unsigned r[24];
        auto pk = [](unsigned lo, unsigned hi) { return (lo & 0xFFFFu) | (hi << 16); };
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // channel ci of position 4t + j: planar f[ci][j]; channels last flat element 3j + ci
            const float v0 = CL ? f[(3 * j) >> 2][(3 * j) & 3] : f[0][j];
            const float v1 = CL ? f[(3 * j + 1) >> 2][(3 * j + 1) & 3] : f[1][j];
            const float v2 = CL ? f[(3 * j + 2) >> 2][(3 * j + 2) & 3] : f[2][j];
            unsigned h01, m01, l01, h2, m2, l2;  // channels 0, 1 packed; channel 2 in the low half
            split3x2(v0, v1, h01, m01, l01);
            split3x2(v2, 0.f, h2, m2, l2);
            r[2 * j] = h01;                          // h0 h1
            r[2 * j + 1] = pk(h2, m01);              // h2 m0
            r[8 + 2 * j] = pk(m01 >> 16, m2);        // m1 m2
            r[8 + 2 * j + 1] = l01;                  // l0 l1
            r[16 + 2 * j] = pk(l2, h01);             // l2 h0
            r[16 + 2 * j + 1] = pk(h01 >> 16, h2);   // h1 h2
        }
        unsigned short* d = ring3 + (z % 3) * k3SlotU + 16 * tid;
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
            *reinterpret_cast<mu4*>(d + sp * k3SplitU) = mu4{r[8 * sp], r[8 * sp + 1], r[8 * sp + 2], r[8 * sp + 3]};
            *reinterpret_cast<mu4*>(d + sp * k3SplitU + 8) = mu4{r[8 * sp + 4], r[8 * sp + 5], r[8 * sp + 6], r[8 * sp + 7]};
        }
    };

    // W (16 x 81) with coalesced loads, then the first run's window behind it (the loads complete
    // in order, so the W staging waits for W alone); eval mode folded in per channel as the
    // fold kernel computes it
    constexpr int WN = 16 * 81, WL = (WN + 255) / 256;
    float wv[WL];
#pragma unroll
    for (int k = 0; k < WL; ++k) {
        const int i = tid + 256 * k;
        wv[k] = i < WN ? w[i] : 0.f;
    }
    float bv = tid < 16 && b ? b[tid] : 0.f;
    if (fold.rv) {
        __shared__ float fold_a3[16];
        if (tid < 16) {
            const float inv = 1.0f / sqrtf(fold.rv[tid] + fold.eps);
            const float gm = fold.gamma ? fold.gamma[tid] : 1.f;
            fold_a3[tid] = gm * inv * fold.scale;
            const float bt = fold.beta ? fold.beta[tid] : 0.f;
            bv = ((bv - fold.rm[tid]) * gm * inv + bt) * fold.scale;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < WL; ++k) {
            const int i = tid + 256 * k;
            if (i < WN) wv[k] = wv[k] * fold_a3[i / 81];
        }
    }
    mf4 rw[3][3];
    if (begin < end) {
        const int64_t sl = begin / k3Tiles, n = sl / OD;
        const int o = (int)(sl - n * OD);
#pragma unroll
        for (int j = 0; j < 3; ++j) fetch(rw[j], n, o + j);
    }
    float* wl = reinterpret_cast<float*>(ring3);  // free until the first window is staged
#pragma unroll
    for (int k = 0; k < WL; ++k) {
        const int i = tid + 256 * k;
        if (i < WN) wl[i] = wv[k];
    }
    if (tid < 16) bias3[tid] = bv;
    __syncthreads();
    // A operands: lane (m, kk) holds row m -- output channel m % 16, part 0 (rows 0..15) or 1
    // (rows 16..31) -- for K elements 8j .. 8j + 7 of its half: element q is element q % 12 of
    // tap k3_tap(kk, q / 12), channel q % 3 of x part (q % 12) / 3 (h, m, l, h), weighted
    // (Wh, Wh, Wh, Wl) in part 0 and (Wm, Wm, Wm, 0) in part 1
    // (each of the lane's 42 weights is read and split once, two at a time by the packed
    // conversion, and fills its 4 elements)
    const int co = m & 15, part = m >> 4;
    bf8 pa[k3Ops];
    {
        unsigned ua[k3Ops * 8];
        auto place = [&](int slot, int ch, unsigned h, unsigned mm, unsigned lo) {
            const int q = 12 * slot + ch;  // x parts h, m, l at q, q + 3, q + 6; h again at q + 9
            ua[q] = ua[q + 3] = ua[q + 6] = (part ? mm : h) & 0xFFFFu;
            ua[q + 9] = part ? 0u : lo & 0xFFFFu;
        };
        auto wt = [&](int slot, int ch) {
            const int tap = k3_tap(kk, slot);
            return tap >= 27 ? 0.f : wl[co * 81 + ch * 27 + tap];
        };
#pragma unroll
        for (int slot = 0; slot < 14; slot += 2) {
            unsigned h, mm, lo;
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                split3x2(wt(slot + d, 0), wt(slot + d, 1), h, mm, lo);
                place(slot + d, 0, h, mm, lo);
                place(slot + d, 1, h >> 16, mm >> 16, lo >> 16);
            }
            split3x2(wt(slot, 2), wt(slot + 1, 2), h, mm, lo);
            place(slot, 2, h, mm, lo);
            place(slot + 1, 2, h >> 16, mm >> 16, lo >> 16);
        }
#pragma unroll
        for (int j = 0; j < k3Ops; ++j)
            pa[j] = __builtin_bit_cast(bf8, mu4{ua[8 * j] | (ua[8 * j + 1] << 16), ua[8 * j + 2] | (ua[8 * j + 3] << 16),
                                                ua[8 * j + 4] | (ua[8 * j + 5] << 16), ua[8 * j + 6] | (ua[8 * j + 7] << 16)});
    }
    mf16 bias16 = {};  // accumulator start: the bias in the upper rows
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        bias16[r] = bias3[4 * kk + r];
        bias16[4 + r] = bias3[8 + 4 * kk + r];
    }
    __syncthreads();  // the W area becomes the first window
    if (begin < end) {
        const int64_t sl = begin / k3Tiles, n = sl / OD;
        const int o = (int)(sl - n * OD);
#pragma unroll
        for (int j = 0; j < 3; ++j) drop(rw[j], o + j);
        __syncthreads();
    }

    // statistics of this lane's 8 channels over the current batch item, one value per channel
    // and tile, by Welford's update with one count for all 8 (they share the positions). The
    // first value becomes the mean exactly (1/1 is exact) and a constant channel adds exact
    // zeros, so it keeps its value as the mean and M2 = 0.
    float mean8[8], m28[8], cnt = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mean8[i] = m28[i] = 0.f;
    auto flush = [&](int64_t n) {
        // The 32 lanes of a half hold the same 8 channels, lanes 0..29 with the same count and
        // lanes 30, 31 with none. Each lane's (count, mean, M2) becomes sums shifted by the
        // mean P of the half's lane 0: S1 = c (mean - P), S2 = M2 + c (mean - P)^2; a butterfly
        // adds them (no divisions), and lane 0 turns the totals back into (count, mean, M2). A
        // constant channel has every mean equal to P, so its sums are exact zeros.
        Stat st[8];
        float P[8], s1[8], s2[8], nt = cnt;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            P[i] = __shfl(mean8[i], l & 32);
            const float d = cnt > 0.f ? mean8[i] - P[i] : 0.f;
            s1[i] = cnt * d;
            s2[i] = fmaf(s1[i], d, m28[i]);
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
            nt += __shfl_xor(nt, off);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                s1[i] += __shfl_xor(s1[i], off);
                s2[i] += __shfl_xor(s2[i], off);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float md = nt > 0.f ? s1[i] / nt : 0.f;
            const float v = s2[i] - s1[i] * md;  // >= 0 but for rounding
            st[i] = nt > 0.f ? Stat{nt, P[i] + md, v < 0.f ? 0.f : v} : stat_empty();
        }
        if (m == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) red3[wave * 16 + (i < 4 ? 4 * kk + i : 4 + 4 * kk + i)] = st[i];
        }
        __syncthreads();
        const int64_t tpn = (int64_t)OD * k3Tiles;
        const int64_t j = wr - ring_wg_of(n * tpn, total, G);
        const bool last = ring_wg_of((n + 1) * tpn - 1, total, G) == wr;
        if (tid < 16) {
            Stat t = red3[tid];
#pragma unroll
            for (int v = 1; v < 4; ++v) t = chan_merge(t, red3[v * 16 + tid]);
            const float pm = rs.pre_mul ? rs.pre_mul[tid] : 1.f;
            float4* slot = rs.part + (n * rs.J) * 16 + tid;
            slot[j * 16] = make_float4(t.n, mul_rn(t.mean, pm), t.m2 * pm * pm, 0.f);
            if (last)
                for (int64_t jj = j + 1; jj < rs.J; ++jj) slot[jj * 16] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();
        cnt = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) mean8[i] = m28[i] = 0.f;
    };

    mf4 pf[3];
    int64_t cur = -1;  // global slice (n * OD + o) whose window is in the ring
    for (int64_t t = begin; t < end;) {
        const int64_t sl = t / k3Tiles;
        const int64_t n = sl / OD;
        const int o = (int)(sl - n * OD);
        const int tlo = (int)(t - sl * k3Tiles);
        const int thi = (int)min((int64_t)k3Tiles, end - sl * k3Tiles);
        if (cur >= 0 && (sl != cur + 1 || o == 0)) {  // a later run: stage its window
#pragma unroll 1
            for (int j = o; j < o + 3; ++j) {
                fetch(pf, n, j);
                drop(pf, j);
            }
            __syncthreads();
        }
        const bool ahead = (sl + 1) * k3Tiles < end && o + 1 < OD;  // the next step continues
        if (ahead) fetch(pf, n, o + 3);

        // this lane's tap rows in this step's window (slot of kd, then kh rows down)
        const int sb0 = (o % 3) * k3SlotU, sb1 = ((o + 1) % 3) * k3SlotU, sb2 = ((o + 2) % 3) * k3SlotU;
        auto rowoff = [&](int R) { return (R < 3 ? sb0 : R < 6 ? sb1 : sb2) + (R % 3) * 32 * 4; };
        int roff[5];
#pragma unroll
        for (int i = 0; i < 4; ++i) roff[i] = kk ? rowoff(4 + i) : rowoff(i);
        // row 8: half 1 reads it two columns right (its kw 2, then the padding tap as kw 3); the
        // lanes past the row (30, 31) stay inside it at column 31
        roff[4] = rowoff(8) + (kk ? (min(m + 2, 31) - m) * 4 : 0);
        // stores through a buffer resource over batch item n's output (16 SP floats; the
        // launcher keeps them below 2^31 bytes): the lane's byte offset in a register, the
        // channel's in a scalar register, so no store needs its own address arithmetic.
        // Planar: channel r (lane half 0) or 4 + r (half 1), then 8 + those, at o * 900 + p;
        // channels last: position o * 900 + p's channels 4kk .. 4kk + 3 and 8 + those.
        const __amdgpu_buffer_rsrc_t cres = __builtin_amdgcn_make_buffer_rsrc(
            c + n * 16 * SP, 0, (int)(16 * SP * 4), 0x00020000 /* 32-bit data format */);
        const uint32_t lane_base = CL ? (uint32_t)(o * k3Pos * 64 + 16 * kk) : (uint32_t)(o * k3Pos * 4) + (kk ? (uint32_t)(16 * SP) : 0u);

        for (int t0 = tlo + 2 * wave; t0 < thi; t0 += 8) {
            int bp[2], p[2];
            bool own[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int ti = t0 + mt;  // output row; ti == thi only as a wave's second tile
                own[mt] = ti < thi && m < 30;
                p[mt] = ti * 30 + m;
                // lanes 30, 31 read input columns 30, 31 (their kw 0), which columns 28, 29
                // take as kw 1, 2 through the lane shift
                bp[mt] = ((ti < 30 ? ti : 29) * 32 + m) * 4;
            }
            mf16 acc[2] = {bias16, bias16};
            // the three areas of a tap row's records at kw 0 (one LDS read each), and at kw + 1
            // by the lane shift
            typedef mu2 Tap[3];
            auto rd = [&](int mt, int i, Tap& k) {
#pragma unroll
                for (int sp = 0; sp < 3; ++sp)
                    k[sp] = *reinterpret_cast<const mu2*>(ring3 + bp[mt] + roff[i] + sp * k3SplitU);
            };
            auto shift = [&](const Tap& a, Tap& b) {
#pragma unroll
                for (int sp = 0; sp < 3; ++sp) b[sp] = mu2{k3_next_lane(a[sp].x), k3_next_lane(a[sp].y)};
            };
            // taps 2s, 2s + 1 of the half's sequence: 24 elements, three instructions
            auto chunk = [&](int s, int mt, const Tap& ta, const Tap& tb) {
                const bf8 b0 = __builtin_bit_cast(bf8, mu4{ta[0].x, ta[0].y, ta[1].x, ta[1].y});
                const bf8 b1 = __builtin_bit_cast(bf8, mu4{ta[2].x, ta[2].y, tb[0].x, tb[0].y});
                const bf8 b2 = __builtin_bit_cast(bf8, mu4{tb[1].x, tb[1].y, tb[2].x, tb[2].y});
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[3 * s], b0, acc[mt], 0, 0, 0);
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[3 * s + 1], b1, acc[mt], 0, 0, 0);
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[3 * s + 2], b2, acc[mt], 0, 0, 0);
            };
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {  // rows 2pr, 2pr + 1 of each half: chunks 3pr .. 3pr + 2
                Tap a0[2], a1[2], a2[2], b0[2], b1[2], b2[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    rd(mt, 2 * pr, a0[mt]);
                    rd(mt, 2 * pr + 1, b0[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    shift(a0[mt], a1[mt]);
                    shift(a1[mt], a2[mt]);
                    shift(b0[mt], b1[mt]);
                    shift(b1[mt], b2[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) chunk(3 * pr, mt, a0[mt], a1[mt]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) chunk(3 * pr + 1, mt, a2[mt], b0[mt]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) chunk(3 * pr + 2, mt, b1[mt], b2[mt]);
            }
            {  // row 8: kw 0, 1 in half 0; kw 2 and the padding tap in half 1 (read 2 columns right)
                Tap c0[2], c1[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) rd(mt, 4, c0[mt]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) shift(c0[mt], c1[mt]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) chunk(6, mt, c0[mt], c1[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                // channels 4kk + r (v[r]) and 8 + 4kk + r (v[4 + r]) at position p
                float v[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = acc[mt][r] + acc[mt][8 + r];
                    v[4 + r] = acc[mt][4 + r] + acc[mt][12 + r];
                }
                if (!own[mt]) continue;
                if (CL) {
                    const int off = (int)(lane_base + 64u * (uint32_t)p[mt]);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(mu4, mf4{v[0], v[1], v[2], v[3]}), cres, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(mu4, mf4{v[4], v[5], v[6], v[7]}), cres, off, 32, 0);
                } else {
                    const int off = (int)(lane_base + 4u * (uint32_t)p[mt]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), cres, off, (int)(r * SP * 4), 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[4 + r]), cres, off, (int)((8 + r) * SP * 4), 0);
                    }
                }
                if (STATS) {
                    cnt += 1.f;
                    const float rn = __builtin_amdgcn_rcpf(cnt);  // 1 ulp; exact at cnt = 1
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float d = v[i] - mean8[i];
                        mean8[i] = fmaf(d, rn, mean8[i]);
                        m28[i] = fmaf(d, v[i] - mean8[i], m28[i]);
                    }
                }
            }
        }
        __syncthreads();  // every wave is done with slot o % 3
        if (ahead) {
            drop(pf, o + 3);
            __syncthreads();
        }
        cur = sl;
        t = (sl + 1) * k3Tiles;
        if (STATS && (t >= end || o + 1 == OD)) flush(n);  // this workgroup's part of item n
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
    float z = ((mul_rn(cv, pm) - s.pivot) - s.mean_d) * A + B;
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
        const f4 cv = cp[k * plane4];  // plain load: the statistics pass just read these lines
        f4 z = ((mul_rn(cv, pm) - s.pivot) - s.mean_d) * A + B;
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

// chain_apply_vec_kernel for instance statistics held in the ring producer's slots: each
// workgroup merges its batch item's slots itself, so no merge launch runs. The values of the
// first kPre channels are loaded before the merge (indexes clamped, so the loads are
// unconditional) and their latency overlaps it.
__global__ __launch_bounds__(kChainBlock) void chain_apply_slots_kernel(ChainArgs a, RingStats rs,
                                                                       float eps)
{
    constexpr int kPre = 8;
    extern __shared__ float coef_raw[];  // [Cout][4]: pm, mean, A, B; then [Cout] post
    float4* coef = reinterpret_cast<float4*>(coef_raw);
    float* post = coef_raw + 4 * a.Cout;
    const int64_t n = blockIdx.y;
    const int64_t i4 = min((int64_t)blockIdx.x * kChainBlock + threadIdx.x, a.SP / 4 - 1);
    const f4* cp = reinterpret_cast<const f4*>(a.c + n * a.Cout * a.SP) + i4;
    const int64_t plane4 = a.SP / 4;
    // R = kChainBlock / Cout adjacent threads per channel (Cout a power of two, 4..256): slot
    // lane r takes slots r, r + R, ... and a butterfly across the R lanes (lower lanes first)
    // merges them, a fixed order. Its loads go out before the data loads (loads complete in
    // order), so the merge waits for them alone.
    const int R = kChainBlock / (int)a.Cout;
    const int kc = threadIdx.x / R, r = threadIdx.x & (R - 1);
    const float4* pp = rs.part + n * rs.J * a.Cout + kc;
    const Stat extra = rs.J > R ? lane_strided_merge_by(rs.J - R, R, [&](int64_t j) {
        const float4 sv = pp[(j + R) * a.Cout];
        return Stat{sv.x, sv.y, sv.z};
    }) : stat_empty();  // slots r + R, r + 2R, ...: only when J > R
    const float4 p0 = pp[min<int64_t>(r, rs.J - 1) * a.Cout];
    const float pm = *(a.pre_mul ? a.pre_mul + kc : &kParamOne);
    const float gm = *(a.gamma ? a.gamma + kc : &kParamOne);
    const float bt = *(a.beta ? a.beta + kc : &kParamZero);
    const float qm = *(a.post_mul ? a.post_mul + kc : &kParamOne);
    f4 v[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) v[k] = cp[min<int64_t>(k, a.Cout - 1) * plane4];
    {
        Stat st = r < rs.J ? Stat{p0.x, p0.y, p0.z} : stat_empty();
        st = chan_merge(st, extra);
        const int lane = threadIdx.x & (kWave - 1);
        for (int off = 1; off < R; off <<= 1) {
            Stat o;
            o.n = __shfl_xor(st.n, off);
            o.mean = __shfl_xor(st.mean, off);
            o.m2 = __shfl_xor(st.m2, off);
            st = (lane & off) ? chan_merge(o, st) : chan_merge(st, o);
        }
        if (r == 0) {
            const float rstd = rsqrtf(st.m2 / st.n + eps);
            coef[kc] = make_float4(pm, st.mean, rstd * gm * a.out_scale, bt * a.out_scale);
            post[kc] = qm;
        }
    }
    __syncthreads();
    if ((int64_t)blockIdx.x * kChainBlock + threadIdx.x >= a.SP / 4) return;
    f4 m = f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    auto one = [&](int k, f4 cv) {
        const float4 q = coef[k];
        f4 z = (mul_rn(cv, q.x) - q.y) * q.z + q.w;
        if (a.clamp) {
            z.x = fminf(fmaxf(z.x, a.lo), a.hi);
            z.y = fminf(fmaxf(z.y, a.lo), a.hi);
            z.z = fminf(fmaxf(z.z, a.lo), a.hi);
            z.w = fminf(fmaxf(z.w, a.lo), a.hi);
        }
        z *= post[k];
        if (a.reduce_max_c) {
            m.x = fmaxf(m.x, z.x);
            m.y = fmaxf(m.y, z.y);
            m.z = fmaxf(m.z, z.z);
            m.w = fmaxf(m.w, z.w);
        } else {
            st_stream(reinterpret_cast<f4*>(a.out + (n * a.Cout + k) * a.SP) + i4, z);
        }
    };
#pragma unroll
    for (int k = 0; k < kPre; ++k)
        if (k < a.Cout) one(k, v[k]);
    for (int k = kPre; k < (int)a.Cout; ++k) one(k, cp[k * plane4]);
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
            const float v = chain_value(a, n, k, a.c[(n * a.Cout + k) * a.SP + i]);
            m = fmaxf(m, v);
        }
        a.out[n * a.SP + i] = m;
    } else {
        for (int64_t k = 0; k < a.Cout; ++k) {
            const int64_t o = (n * a.Cout + k) * a.SP + i;
            a.out[o] = chain_value(a, n, k, a.c[o]);
        }
    }
}

}  // namespace

namespace {
bool conv_valu_forced()
{
    const char* e = getenv("NORMRED_CONV");
    return e && e[0] == 'v';  // "valu": the vector-ALU producer (comparisons)
}

bool conv_fp32_forced()
{
    const char* e = getenv("NORMRED_CONV");
    return e && e[0] == 'f';  // "fp32": the 2-D producer on the fp32 matrix instruction
}

constexpr int kRingLdsMax = 64 * 1024;  // LDS bytes of one workgroup's ring

// Ring geometry for the persistent producer; false when the shape does not fit (ring beyond
// kRingLdsMax, one input slice beyond PF float4 per thread, or offsets beyond 24 bits).
bool make_ring(const ConvGeom& g, const float* x, const float* c, int PF, ConvRing* rg)
{
    const bool d3 = g.dims == 3;
    rg->OO = (int)(d3 ? g.OD : g.OH);
    rg->outer_in = (int)(d3 ? g.D : g.H);
    rg->inner_in = (int)(d3 ? g.H * g.W : g.W);
    rg->inner_out = (int)(d3 ? g.OH * g.OW : g.OW);
    const int64_t slice = g.Cin * (int64_t)rg->inner_in;
    if (4 * slice * (int64_t)sizeof(float) > kRingLdsMax) return false;
    if (slice > 4LL * PF * kMfmaBlock || 4 * slice >= (1 << 24)) return false;
    if (g.cl) {
        // a slice is one contiguous run; a lane stores 4 consecutive channels of a position
        rg->vec_in = (slice % 4 == 0) && ((uintptr_t)x % 16 == 0);
        rg->vec_out = (g.Cout % 4 == 0) && ((uintptr_t)c % 16 == 0);
        rg->T = (rg->inner_out + 15) / 16;
        return true;
    }
    rg->vec_in = (rg->inner_in % 4 == 0) && ((uintptr_t)x % 16 == 0);
    rg->vec_out = (g.SP % 4 == 0) && ((uintptr_t)c % 16 == 0);
    // largest start shift of a slice's tiles: 0 when a slice is a multiple of 4 positions,
    // 2 when it is even, else 3
    const int maxshift = !rg->vec_out ? 0 : rg->inner_out % 4 == 0 ? 0 : rg->inner_out % 2 == 0 ? 2 : 3;
    rg->T = (rg->inner_out + maxshift + 15) / 16;
    return true;
}

// Compute units of the current device (the runtime caches device attributes).
int device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 256;
    return cus;
}

int ring_grid(const ConvGeom& g, const ConvRing& rg, int wgs_per_cu)
{
    const int cus = device_cus();
    if (const char* e = getenv("NORMRED_CONV_WGS_PER_CU")) wgs_per_cu = std::max(1, atoi(e));
    const int64_t total = g.N * (int64_t)rg.OO * rg.T;
    return (int)std::max<int64_t>(1, std::min<int64_t>(total, (int64_t)cus * wgs_per_cu));
}

template <int DIMS, int KS, int WAVES_N, int MT, int PF>
hipError_t launch_ring(const ConvGeom& g, const ConvRing& rg, int wgs_per_cu, const float* x,
                       const float* w, const float* b, float* c, const RingStats* rs,
                       hipStream_t stream, const ConvFold* fold = nullptr)
{
    // the ring, which first holds W (C_out x K floats) and the bias while the lanes take theirs;
    // with statistics, one Stat per (wave row, channel) after it; then the tap table
    constexpr int WAVES_M = (kMfmaBlock / 64) / WAVES_N;
    const size_t lds = (size_t)ring_main_floats(g, rg, DIMS) * sizeof(float) +
                       (rs ? (size_t)WAVES_M * g.Cout * sizeof(Stat) : 0) + 4 * KS * sizeof(int);
    const int grid = ring_grid(g, rg, wgs_per_cu);
    const dim3 gd(grid), bd(kMfmaBlock);
    const RingStats none{nullptr, nullptr, 0};
    const ConvFold nofold{nullptr, nullptr, nullptr, nullptr, 0.f, 1.f};
    const ConvFold fd = fold ? *fold : nofold;
    // 3-D input planes of 32 x 32 (the IN3d model's) take a copy with the plane extents as
    // constants: its per-tile position arithmetic is a multiply and shift (2-3 % faster)
    const bool p32 = DIMS == 3 && g.W == 32 && g.H == 32;
#define NR_RING(VEC, CL, ST)                                                                     \
    do {                                                                                         \
        if (p32 && VEC)                                                                          \
            conv_k3_ring_kernel<DIMS, KS, WAVES_N, MT, PF, VEC, CL, ST, DIMS == 3><<<gd, bd, lds, stream>>>( \
                g, rg, x, w, b, c, rs ? *rs : none, fd);                                         \
        else                                                                                     \
            conv_k3_ring_kernel<DIMS, KS, WAVES_N, MT, PF, VEC, CL, ST><<<gd, bd, lds, stream>>>( \
                g, rg, x, w, b, c, rs ? *rs : none, fd);                                         \
    } while (0)
    if (rs) {
        if (g.cl && rg.vec_in)
            NR_RING(true, true, true);
        else if (g.cl)
            NR_RING(false, true, true);
        else if (rg.vec_in)
            NR_RING(true, false, true);
        else
            NR_RING(false, false, true);
    } else {
        if (g.cl && rg.vec_in)
            NR_RING(true, true, false);
        else if (g.cl)
            NR_RING(false, true, false);
        else if (rg.vec_in)
            NR_RING(true, false, false);
        else
            NR_RING(false, false, false);
    }
#undef NR_RING
    return hipGetLastError();
}

// The shapes the ring producer is compiled for: 2-D C_in 8 -> C_out 64 and 3-D C_in 3 -> 16,
// with int32 offsets into one batch item.
enum RingShape { kRingNone, kRing2d, kRing3d };
constexpr int kRingWgs2d = 4, kRingWgs3d = 3;  // workgroups per CU of the two ring producers
constexpr int kRingWgsStats = 3;                // either, taking statistics
constexpr int64_t kRingMaxSlots = 128;          // statistics slots per batch item, at most
RingShape ring_shape(const ConvGeom& g)
{
    const bool small = g.Cin * g.D * g.H * g.W < (1LL << 31) && g.SP < (1LL << 31);
    if (!small || conv_valu_forced()) return kRingNone;
    if (g.dims == 2 && g.Cin == 8 && g.Cout == 64) return kRing2d;
    if (g.dims == 3 && g.Cin == 3 && g.Cout == 16) return kRing3d;
    return kRingNone;
}

constexpr int kC8B = 4;  // output rows per box of the 2-D matrix producer (2 measured ~8 % slower)

// Persistent grid of the 2-D matrix producer: two workgroups per CU (one wave per SIMD each,
// the most its VGPR use allows), at most one per box.
int64_t c8_grid(const ConvGeom& g)
{
    int wgs = 2;
    if (const char* e = getenv("NORMRED_CONV_WGS_PER_CU")) wgs = std::min(8, std::max(1, atoi(e)));
    const int64_t nbox = (g.OH + kC8B - 1) / kC8B;
    return std::min<int64_t>(std::min<int64_t>(g.N * nbox, (int64_t)device_cus() * wgs), kC8MaxGrid);
}

// The 3-D bf16 producer's shape: C_in 3 -> C_out 16 over 32 x 32 input planes.
bool conv3d_c3_shape(const ConvGeom& g)
{
    return g.dims == 3 && g.Cin == 3 && g.Cout == 16 && g.H == 32 && g.W == 32 && g.D >= 3 &&
           g.SP * 16 * 4 < (1LL << 31);
}

// ... and a call it takes: x and the output 16-byte aligned (its staging loads and
// channels-last stores are 16-byte vectors); NORMRED_CONV=fp32 or valu picks the others.
bool conv3d_c3_ok(const ConvGeom& g, const void* x, const void* c)
{
    return conv3d_c3_shape(g) && !conv_valu_forced() && !conv_fp32_forced() &&
           ((uintptr_t)x | (uintptr_t)c) % 16 == 0;
}

int64_t c3_grid(const ConvGeom& g)
{
    int wgs = k3Wgs;
    if (const char* e = getenv("NORMRED_CONV_WGS_PER_CU")) wgs = std::min(8, std::max(1, atoi(e)));
    return std::max<int64_t>(1, std::min<int64_t>(g.N * g.OD * k3Tiles, (int64_t)device_cus() * wgs));
}

// Statistics slots per batch item of the 3-D bf16 producer (the bound of ring_slots_for).
int64_t c3_slots(const ConvGeom& g)
{
    const int64_t L = g.OD * k3Tiles, total = g.N * L, m = total / c3_grid(g);
    return L < 2 ? 1 : (L - 2) / m + 2;
}

hipError_t launch_conv3d_c3(const ConvGeom& g, const float* x, const float* w, const float* b,
                            float* c, const RingStats* rs, const ConvFold* fold, hipStream_t stream)
{
    const dim3 gd((unsigned)c3_grid(g)), bd(256);
    const RingStats none{nullptr, nullptr, 0};
    const ConvFold nofold{nullptr, nullptr, nullptr, nullptr, 0.f, 1.f};
    const RingStats r = rs ? *rs : none;
    const ConvFold fd = fold ? *fold : nofold;
    if (rs && g.cl)
        conv3d_c3_bf16x6_kernel<true, true><<<gd, bd, 0, stream>>>(g, x, w, b, c, r, fd);
    else if (rs)
        conv3d_c3_bf16x6_kernel<false, true><<<gd, bd, 0, stream>>>(g, x, w, b, c, r, fd);
    else if (g.cl)
        conv3d_c3_bf16x6_kernel<true, false><<<gd, bd, 0, stream>>>(g, x, w, b, c, r, fd);
    else
        conv3d_c3_bf16x6_kernel<false, false><<<gd, bd, 0, stream>>>(g, x, w, b, c, r, fd);
    return hipGetLastError();
}
}  // namespace

// 16-byte output stores need every box to start on a multiple of 4 positions: kC8B * 62 is,
// and SP % 4 == 0 keeps planes aligned. SP % 4 == 0 also means an even output height, so every
// box holds an even number of rows (at least 124 positions, a multiple of 4).
bool conv2d_c8_shape(const ConvGeom& g)
{
    return !g.cl && g.dims == 2 && g.Cin == kC8Cin && g.Cout == kC8Cout && g.W == kC8W &&
           g.SP % 4 == 0 && g.Cin * g.D * g.H * g.W < (1LL << 31) && g.SP * kC8Cout * 4 < (1LL << 31);
}

int64_t conv2d_c8_stats_grid(const ConvGeom& g) { return c8_grid(g); }

int64_t conv2d_c8_grid_bound(const ConvGeom& g)
{
    return std::min<int64_t>(g.N * ((g.OH + kC8B - 1) / kC8B), kC8MaxGrid);
}

bool conv2d_c8_recompute(const ConvGeom& g, const void* x, const void* out)
{
    return conv2d_c8_shape(g) && !conv_valu_forced() && !conv_fp32_forced() &&
           (uintptr_t)x % 16 == 0 && (uintptr_t)out % 16 == 0;
}

// Two launches of the same grid: the statistics pass (partials per workgroup and channel; its
// workgroup 0 clears the words the merge publishes), then the apply pass, whose first
// workgroups merge one channel each before their own work. The apply pass's workgroups wait
// only on workgroups that start before them (the lowest-numbered), which therefore run.
hipError_t launch_conv2d_c8_bn_chain(const ConvGeom& g, const float* x, const float* w,
                                     const float* b, float* out, C8Chain e, hipStream_t stream)
{
    const int64_t G = c8_grid(g);
    e.nparts = (int)G;
    // NORMRED_TEST_WAIT_GIVEUP=1 (tests of the failure path only), as for the read-once kernels:
    // the wait looks for a tag nothing publishes and gives up after 64 polls
    const char* giveup = getenv("NORMRED_TEST_WAIT_GIVEUP");
    const bool test_giveup = giveup && giveup[0] == '1';
    e.wait_tag = test_giveup ? kC8Tag + 1u : kC8Tag;
    e.spin_limit = test_giveup ? 64u : kSpinLimit;
    conv2d_c8_bf16x6_kernel<kC8B, kC8Stats><<<dim3((unsigned)G), dim3(256), 0, stream>>>(g, x, w, b, nullptr, e);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (!e.pre_mul && !e.clamp && !e.post_mul)
        conv2d_c8_bf16x6_kernel<kC8B, kC8ApplyPlain><<<dim3((unsigned)G), dim3(256), 0, stream>>>(g, x, w, b, out, e);
    else
        conv2d_c8_bf16x6_kernel<kC8B, kC8Apply><<<dim3((unsigned)G), dim3(256), 0, stream>>>(g, x, w, b, out, e);
    return hipGetLastError();
}

bool conv_k3_eval_direct_ok(const ConvGeom& g, const void* x, const void* out)
{
    const bool small = g.Cin * g.D * g.H * g.W < (1LL << 31) && g.SP < (1LL << 31);
    if (!small || conv_valu_forced()) return false;
    if (conv2d_c8_shape(g))
        return !conv_fp32_forced() && (uintptr_t)x % 16 == 0 && (uintptr_t)out % 16 == 0;
    if (conv3d_c3_ok(g, x, out)) return true;
    ConvRing rg;
    const RingShape shape = ring_shape(g);
    return (shape == kRing2d && make_ring(g, (const float*)x, (const float*)out, 1, &rg)) ||
           (shape == kRing3d && make_ring(g, (const float*)x, (const float*)out, 3, &rg));
}

hipError_t launch_conv_k3_eval(const ConvGeom& g, const float* x, const float* w, const float* b,
                               const ConvFold& fold, float* out, hipStream_t stream)
{
    if (!conv_k3_eval_direct_ok(g, x, out)) return hipErrorInvalidValue;
    if (conv2d_c8_shape(g)) {
        C8Chain e;
        e.fold_rm = fold.rm;
        e.fold_rv = fold.rv;
        e.gamma = fold.gamma;
        e.beta = fold.beta;
        e.eps = fold.eps;
        e.out_scale = fold.scale;
        conv2d_c8_bf16x6_kernel<kC8B, kC8Conv><<<dim3((unsigned)c8_grid(g)), dim3(256), 0, stream>>>(
            g, x, w, b, out, e);
        return hipGetLastError();
    }
    if (conv3d_c3_ok(g, x, out)) return launch_conv3d_c3(g, x, w, b, out, nullptr, &fold, stream);
    ConvRing rg;
    if (ring_shape(g) == kRing2d && make_ring(g, x, out, 1, &rg))
        return launch_ring<2, 18, 4, 4, 1>(g, rg, kRingWgs2d, x, w, b, out, nullptr, stream, &fold);
    if (ring_shape(g) == kRing3d && make_ring(g, x, out, 3, &rg))
        return launch_ring<3, 21, 1, 2, 3>(g, rg, kRingWgs3d, x, w, b, out, nullptr, stream, &fold);
    return hipErrorInvalidValue;
}

hipError_t launch_conv_k3(const ConvGeom& g, const float* x, const float* w, const float* b,
                          float* c, hipStream_t stream)
{
    // Matrix-core producers for the compiled (dims, C_in, C_out) shapes; int32 offsets into one
    // batch item of x.
    const bool small = g.Cin * g.D * g.H * g.W < (1LL << 31) && g.SP < (1LL << 31);
    ConvRing rg;
    if (!conv_valu_forced() && small) {
        // 16-byte output stores need every box to start on a multiple of 4 positions: B * 62
        // is, SP % 4 == 0 keeps planes aligned. SP % 4 == 0 also means an even output height,
        // so every box holds an even number of rows (at least 124 positions, a multiple of 4)
        if (conv2d_c8_shape(g) && (uintptr_t)x % 16 == 0 && (uintptr_t)c % 16 == 0) {
            const int64_t grid = c8_grid(g);
            if (conv_fp32_forced())
                conv2d_c8_mfma32_kernel<kC8B><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(g, x, w, b, c);
            else
                conv2d_c8_bf16x6_kernel<kC8B, kC8Conv><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
                    g, x, w, b, c, C8Chain{});
            return hipGetLastError();
        }
        if (ring_shape(g) == kRing2d && make_ring(g, x, c, 1, &rg))
            return launch_ring<2, 18, 4, 4, 1>(g, rg, kRingWgs2d, x, w, b, c, nullptr, stream);
        if (conv3d_c3_ok(g, x, c)) return launch_conv3d_c3(g, x, w, b, c, nullptr, nullptr, stream);
        if (ring_shape(g) == kRing3d && make_ring(g, x, c, 3, &rg))
            return launch_ring<3, 21, 1, 2, 3>(g, rg, kRingWgs3d, x, w, b, c, nullptr, stream);
    }
    const dim3 grid((unsigned)((g.SP + kConvBlock - 1) / kConvBlock), (unsigned)g.N,
                    (unsigned)((g.Cout + kKB - 1) / kKB));
    if (g.dims == 3 && g.cl)
        conv_k3_kernel<3, true><<<grid, dim3(kConvBlock), 0, stream>>>(g, x, w, b, c);
    else if (g.dims == 3)
        conv_k3_kernel<3, false><<<grid, dim3(kConvBlock), 0, stream>>>(g, x, w, b, c);
    else if (g.cl)
        conv_k3_kernel<2, true><<<grid, dim3(kConvBlock), 0, stream>>>(g, x, w, b, c);
    else
        conv_k3_kernel<2, false><<<grid, dim3(kConvBlock), 0, stream>>>(g, x, w, b, c);
    return hipGetLastError();
}

hipError_t launch_chain_apply_slots(const ChainArgs& a, const RingStats& rs, float eps,
                                   hipStream_t stream)
{
    const int64_t n4 = a.SP / 4;
    const dim3 grid((unsigned)((n4 + kChainBlock - 1) / kChainBlock), (unsigned)a.N);
    const size_t lds = (size_t)a.Cout * 5 * sizeof(float);
    chain_apply_slots_kernel<<<grid, dim3(kChainBlock), lds, stream>>>(a, rs, eps);
    return hipGetLastError();
}

bool chain_apply_slots_ok(const ChainArgs& a)
{
    return (a.SP & 3) == 0 && !a.batch && a.Cout >= 4 && a.Cout <= kChainBlock &&
           (a.Cout & (a.Cout - 1)) == 0 &&
           ((reinterpret_cast<uintptr_t>(a.c) | reinterpret_cast<uintptr_t>(a.out)) & 15) == 0;
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

namespace nr {
namespace {

// Slots for one tile count per slice: at most floor((L - 2) / m) + 2 workgroups meet a run of
// L >= 2 tiles when every workgroup range holds at least m tiles (the first and last meet it
// with a tile each, the others lie inside it).
int64_t ring_slots_for(const ConvGeom& g, const ConvRing& rg, int wgs)
{
    const int64_t L = (int64_t)rg.OO * rg.T;
    const int64_t total = g.N * L;
    const int64_t G = ring_grid(g, rg, wgs);
    const int64_t m = total / G;  // >= 1: the grid never exceeds the tiles
    return L < 2 ? 1 : (L - 2) / m + 2;
}

__global__ __launch_bounds__(256) void ring_stats_merge_kernel(RingStats rs, int64_t N, int64_t C,
                                                               float eps, GroupStat* __restrict__ stats)
{
    const int64_t grp = (int64_t)blockIdx.x * 256 + threadIdx.x;  // n * C + k
    if (grp >= N * C) return;
    const int64_t n = grp / C, k = grp - n * C;
    const float4* pp = rs.part + n * rs.J * C + k;
    Stat st = stat_empty();
    for (int64_t j = 0; j < rs.J; ++j) {
        const float4 v = pp[j * C];
        st = chan_merge(st, Stat{v.x, v.y, v.z});
    }
    stats[grp] = GroupStat{0.f, st.mean, rsqrtf(st.m2 / st.n + eps), 0.f};
}
}  // namespace

int64_t ring_stats_slots(const ConvGeom& g)
{
    const RingShape shape = ring_shape(g);
    // the 2-D 64-wide shape keeps its own producer (faster than the ring)
    if (shape == kRingNone || g.N == 0 || conv2d_c8_shape(g)) return 0;
    // the tile count per slice depends on the output's alignment (planar): take the most slots
    // over the alignments a call may bring
    alignas(16) static const float probe[4] = {0.f, 0.f, 0.f, 0.f};
    const int PF = shape == kRing2d ? 1 : 3;
    int64_t J = 0;
    for (int mis = 0; mis < 4; ++mis) {
        ConvRing rg;
        if (!make_ring(g, probe, probe + mis, PF, &rg)) return 0;
        J = std::max(J, ring_slots_for(g, rg, kRingWgsStats));
    }
    if (conv3d_c3_shape(g)) J = std::max(J, c3_slots(g));  // the 3-D bf16 producer's slots
    // small batches spread an item over many workgroups: past kRingMaxSlots slots the epilogue
    // workgroups would spend longer merging them than a statistics pass over c takes
    return J <= kRingMaxSlots ? J : 0;
}

hipError_t launch_conv_k3_stats(const ConvGeom& g, const float* x, const float* w, const float* b,
                                float* c, RingStats rs, hipStream_t stream)
{
    if (conv3d_c3_ok(g, x, c) && c3_slots(g) <= rs.J)
        return launch_conv3d_c3(g, x, w, b, c, &rs, nullptr, stream);
    const RingShape shape = ring_shape(g);
    ConvRing rg;
    if (shape == kRing2d && make_ring(g, x, c, 1, &rg) && ring_slots_for(g, rg, kRingWgsStats) <= rs.J)
        return launch_ring<2, 18, 4, 4, 1>(g, rg, kRingWgsStats, x, w, b, c, &rs, stream);
    if (shape == kRing3d && make_ring(g, x, c, 3, &rg) && ring_slots_for(g, rg, kRingWgsStats) <= rs.J)
        return launch_ring<3, 21, 1, 2, 3>(g, rg, kRingWgsStats, x, w, b, c, &rs, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_ring_stats_merge(const ConvGeom& g, const RingStats& rs, float eps,
                                   GroupStat* stats, hipStream_t stream)
{
    const int64_t groups = g.N * g.Cout;
    ring_stats_merge_kernel<<<dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream>>>(
        rs, g.N, g.Cout, eps, stats);
    return hipGetLastError();
}
}  // namespace nr
