// stats_split.hip -- streaming statistics for any slice length or alignment, and for batch
// normalization, on gfx950.
//
// Operations: IN2d page (task l1_p34), statement of the op (instance statistics per (n, c));
// BN page (task l2_p73), opening analysis (training-mode batch statistics per channel over
// (n, h, w)). Both reduce to "mean and biased variance of a group of slices": a group is one
// slice for instance norm and the N slices of one channel for batch norm.
//
// Three kernels, each deterministic:
//   1. partial: one workgroup per (slice, chunk) streams its chunk once and writes the chunk's
//      (mean, M2) relative to the group's pivot. Per thread, values are taken 16 at a time from
//      16-byte loads, reduced by the two-pass formula over registers and folded into a running
//      state with the pairwise (Chan) merge -- the batched form of the per-element Welford
//      update both pages use, with one division per 16 values instead of one per value.
//   2. merge: one wave per group merges all of the group's chunk partials in a fixed order
//      (the page's split-slice scheme with a final fixed-order combine instead of float
//      atomics) and writes pivot, mean - pivot and 1/sqrt(var + eps).
//   3. apply: one workgroup per (slice, chunk) normalizes its chunk (second read of x).
// Slices that do not start on 16-byte boundaries (S not a multiple of 4) in 16-byte aligned
// tensors take flat variants of the partial and apply steps that keep 16-byte accesses: the
// partial step gives each (slice, chunk) one wave, which reads the aligned 16-byte blocks
// covering its range and masks the values outside it (reading a neighbour's edge values does
// no harm); the apply step walks the whole tensor in aligned blocks, and each value takes the
// coefficients of its own slice, so a block that straddles two slices is written whole and
// right. Only the tensor's last block, when it is partial, uses 4-byte accesses.
#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

constexpr int kBlock = 256;
constexpr int kNW = kBlock / kWave;

__device__ __forceinline__ int64_t chunk_len(const SplitGeom& g, int64_t ch)
{
    const int64_t r = g.S - ch * g.chunk;
    return r < g.chunk ? r : g.chunk;
}

// Index of the slice holding a group's pivot (its first element).
// (instance: the slice itself; batch: channel c's first slice, n = 0, has index c)
__device__ __forceinline__ int64_t pivot_slice(int64_t group) { return group; }

__device__ __forceinline__ int64_t group_of(const SplitGeom& g, int64_t slice)
{
    return g.batch ? slice % g.C : slice;
}

// Fold a batch of values into a running state. d[0..n) hold the (pivot-shifted) values and
// d[n..16) are zero; indices are static so the batch stays in registers.
__device__ __forceinline__ Stat fold16(Stat run, const float (&d)[16], int n)
{
    if (n <= 0) return run;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += d[i];
    const float fn = (float)n;
    const float m = s / fn;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i < n) q = fmaf(d[i] - m, d[i] - m, q);
    return chan_merge(run, Stat{fn, m, q});
}

// CACHED: plain loads instead of streaming ones, for a chain's conv output that the epilogue
// reads again right after (measured: the epilogue pass 20.8 -> 17.0 us on the IN3d workload).
// FINAL: instance groups of one chunk, whose partial is the group's statistics: write them as
// the merge step would (same arithmetic: merging one partial with empty ones changes nothing)
// and skip the merge launch.
template <bool VEC, bool CACHED, bool FINAL>
__global__ __launch_bounds__(kBlock) void split_partial_kernel(SplitGeom g, const float* x,
                                                               const float* pre_mul,
                                                               float2* partials, float eps,
                                                               GroupStat* stats, float* save_mean,
                                                               float* save_invstd)
{
    __shared__ Stat wstat[kNW];
    const int64_t wg = blockIdx.x;
    const int64_t slice = wg / g.chunks;
    const int64_t ch = wg - slice * g.chunks;
    const int64_t c = slice % g.C;
    const float m = pre_mul ? pre_mul[c] : 1.f;
    const float K = mul_rn(x[pivot_slice(group_of(g, slice)) * g.S], m);
    const int64_t start = ch * g.chunk;
    const int64_t len = chunk_len(g, ch);
    const float* xs = x + slice * g.S + start;
    const int tid = threadIdx.x;

    Stat st = stat_empty();
    float d[16];
    if (VEC) {
        const f4* xv = reinterpret_cast<const f4*>(xs);
        const int64_t nv = len >> 2;
        for (int64_t i0 = 0; i0 < nv; i0 += 4 * kBlock) {
            int n = 0;  // valid entries form a prefix: j < some bound
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = i0 + j * kBlock + tid;
                f4 t = f4{0.f, 0.f, 0.f, 0.f};
                if (i < nv) {
                    t = mul_rn(CACHED ? xv[i] : ld_stream(xv + i), m) - K;
                    n += 4;
                }
                d[4 * j + 0] = t.x;
                d[4 * j + 1] = t.y;
                d[4 * j + 2] = t.z;
                d[4 * j + 3] = t.w;
            }
            st = fold16(st, d, n);
        }
    } else {
        for (int64_t i0 = 0; i0 < len; i0 += 16 * kBlock) {
            int n = 0;  // valid entries form a prefix
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t i = i0 + j * kBlock + tid;
                d[j] = 0.f;
                if (i < len) {
                    d[j] = mul_rn(CACHED ? xs[i] : ld_stream1(xs + i), m) - K;
                    ++n;
                }
            }
            st = fold16(st, d, n);
        }
    }

    st = wave_merge<kWave>(st);
    if (lane_id() == 0) wstat[tid / kWave] = st;
    __syncthreads();
    if (tid < kWave) {
        Stat w = tid < kNW ? wstat[tid] : stat_empty();
        w = wave_merge<kNW>(w);
        if (tid == 0) {
            if (FINAL) {
                const float rstd = rsqrtf(w.m2 / w.n + eps);
                stats[slice] = GroupStat{K, w.mean, rstd, 0.f};
                if (save_mean) save_mean[slice] = K + w.mean;
                if (save_invstd) save_invstd[slice] = rstd;
            } else {
                partials[wg] = make_float2(w.mean, w.m2);
            }
        }
    }
}

// One wave per group.
__global__ __launch_bounds__(kWave) void split_merge_kernel(SplitGeom g, const float* x,
                                                            const float* pre_mul,
                                                            const float2* partials, float eps,
                                                            GroupStat* stats, float* save_mean,
                                                            float* save_invstd, RunningStats run)
{
    const int64_t grp = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t members = g.batch ? g.slices / g.C : 1;
    const int64_t total = members * g.chunks;

    Stat st = lane_strided_merge<kWave>(total, [&](int64_t q) {
        const int64_t mem = q / g.chunks;
        const int64_t ch = q - mem * g.chunks;
        const int64_t slice = g.batch ? mem * g.C + grp : grp;
        const float2 p = partials[slice * g.chunks + ch];
        return Stat{(float)chunk_len(g, ch), p.x, p.y};
    });
    st = wave_merge<kWave>(st);
    if (lane == 0) {
        const int64_t c = grp % g.C;
        const float m = pre_mul ? pre_mul[c] : 1.f;
        const float K = mul_rn(x[pivot_slice(grp) * g.S], m);
        const float rstd = rsqrtf(st.m2 / st.n + eps);
        stats[grp] = GroupStat{K, st.mean, rstd, 0.f};
        if (save_mean) save_mean[grp] = K + st.mean;
        if (save_invstd) save_invstd[grp] = rstd;
        if (run.mean) {
            // BN page, opening analysis: running = (1 - m) * running + m * batch, with the
            // unbiased batch variance
            const float m = run.momentum;
            run.mean[grp] = (1.f - m) * run.mean[grp] + m * (K + st.mean);
            run.var[grp] = (1.f - m) * run.var[grp] + m * (st.m2 / (st.n - 1.f));
        }
    }
}

// Flat partial step: one aligned group of LANES lanes (4..64) per (slice, chunk) unit,
// kBlock / LANES units per workgroup (unit u = slice * chunks + chunk, as the partial index);
// short units take narrow groups so that few lanes idle. x is 16-byte aligned;
// T = slices * S < 2^32.
template <bool CACHED, bool FINAL, int LANES>
__global__ __launch_bounds__(kBlock) void split_partial_flat_kernel(SplitGeom g, const float* x,
                                                                    const float* pre_mul,
                                                                    float2* partials, float eps,
                                                                    GroupStat* stats,
                                                                    float* save_mean,
                                                                    float* save_invstd, int64_t units)
{
    const int lane = threadIdx.x & (LANES - 1);
    const int64_t u = (int64_t)blockIdx.x * (kBlock / LANES) + threadIdx.x / LANES;
    if (u >= units) return;  // whole groups only: no barrier, and shuffles stay in the group
    const int64_t slice = u / g.chunks;
    const int64_t ch = u - slice * g.chunks;
    const int64_t c = slice % g.C;
    const float m = pre_mul ? pre_mul[c] : 1.f;
    const float K = mul_rn(x[pivot_slice(group_of(g, slice)) * g.S], m);
    const int64_t T = g.slices * g.S;
    const int64_t start = slice * g.S + ch * g.chunk;
    const int64_t end = start + chunk_len(g, ch);
    const int64_t b_lo = start >> 2, b_hi = (end + 3) >> 2;  // aligned blocks covering the unit
    const f4* xv = reinterpret_cast<const f4*>(x);
    Stat st = stat_empty();
    for (int64_t b0 = b_lo; b0 < b_hi; b0 += 4 * LANES) {
        float d[16];
        bool in[16];
        int n = 0;
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t b = b0 + j * LANES + lane;
            f4 v = f4{0.f, 0.f, 0.f, 0.f};
            if (b < b_hi) {
                if (4 * b + 3 < T) {
                    v = CACHED ? xv[b] : ld_stream(xv + b);
                } else {  // the tensor's last, partial block
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * b + e < T) v[e] = CACHED ? x[4 * b + e] : ld_stream1(x + 4 * b + e);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t i = 4 * b + e;
                const bool ok = b < b_hi && i >= start && i < end;
                in[4 * j + e] = ok;
                d[4 * j + e] = ok ? mul_rn(v[e], m) - K : 0.f;
                n += ok;
                sum += d[4 * j + e];
            }
        }
        if (n > 0) {
            const float fn = (float)n, mean = sum / fn;
            float q = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (in[i]) q = fmaf(d[i] - mean, d[i] - mean, q);
            st = chan_merge(st, Stat{fn, mean, q});
        }
    }
    st = wave_merge<LANES>(st);
    if (lane == 0) {
        if (FINAL) {
            const float rstd = rsqrtf(st.m2 / st.n + eps);
            stats[slice] = GroupStat{K, st.mean, rstd, 0.f};
            if (save_mean) save_mean[slice] = K + st.mean;
            if (save_invstd) save_invstd[slice] = rstd;
        } else {
            partials[u] = make_float2(st.mean, st.m2);
        }
    }
}

// Flat apply step: thread -> one aligned 16-byte block of the whole tensor (dealt so that each
// XCD streams a contiguous eighth, as split_apply_vec_kernel); each value takes its own
// slice's coefficients. x and y are 16-byte aligned; T = slices * S < 2^32.
__global__ __launch_bounds__(kBlock) void split_apply_flat_kernel(SplitGeom g, const float* x,
                                                                  float* y, const GroupStat* stats,
                                                                  const float* gamma,
                                                                  const float* beta,
                                                                  float out_scale, int64_t nblocks)
{
    int64_t w = blockIdx.x;
    const int64_t wgs = gridDim.x, w8 = wgs / 8 * 8;
    if (w < w8) w = (w % 8) * (w8 / 8) + w / 8;
    const int64_t b = w * kBlock + threadIdx.x;
    if (b >= nblocks) return;
    const uint32_t T = (uint32_t)(g.slices * g.S), S = (uint32_t)g.S;
    const uint32_t e0 = (uint32_t)(4 * b);
    const bool whole = e0 + 3 < T;
    f4 v = f4{0.f, 0.f, 0.f, 0.f};
    if (whole) {
        v = ld_stream(reinterpret_cast<const f4*>(x) + b);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e0 + e < T) v[e] = ld_stream1(x + e0 + e);
    }
    uint32_t sl = e0 / S, r = e0 - sl * S;  // slice and offset of the block's first value
    f4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        while (r >= S) {  // at most 3 steps: the block holds 4 values
            r -= S;
            ++sl;
        }
        const int64_t slice = sl < (uint32_t)g.slices ? sl : g.slices - 1;  // tail past T
        const int64_t c = slice % g.C;
        const GroupStat st = stats[group_of(g, slice)];
        const float A = st.rstd * (gamma ? gamma[c] : 1.f) * out_scale;
        const float B = (beta ? beta[c] : 0.f) * out_scale;
        z[e] = ((v[e] - st.pivot) - st.mean_d) * A + B;
        ++r;
    }
    if (whole) {
        st_stream(reinterpret_cast<f4*>(y) + b, z);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e0 + e < T) st_stream1(y + e0 + e, z[e]);
    }
}

// Normalize pass, 16-byte path: one 1024-value sub-chunk of one slice per workgroup (one
// vector per thread), a one-shot grid dealt so that each XCD streams a contiguous eighth of
// the sub-chunks -- the fastest streaming pattern measured on MI355X.
__global__ __launch_bounds__(kBlock) void split_apply_vec_kernel(SplitGeom g, const float* x, float* y,
                                                                 const GroupStat* stats,
                                                                 const float* gamma,
                                                                 const float* beta, float out_scale,
                                                                 int64_t subs, int64_t total)
{
    int64_t b = blockIdx.x;
    const int64_t t8 = total / 8 * 8;
    if (b < t8) b = (b % 8) * (t8 / 8) + b / 8;
    const int64_t slice = b / subs;
    const int64_t sub = b - slice * subs;
    const int64_t c = slice % g.C;
    const GroupStat s = stats[group_of(g, slice)];
    const float A = s.rstd * (gamma ? gamma[c] : 1.f) * out_scale;
    const float B = (beta ? beta[c] : 0.f) * out_scale;
    const int64_t i = sub * (4 * kBlock) + 4 * threadIdx.x;  // value index in the slice
    if (i >= g.S) return;
    const int64_t off = slice * g.S + i;
    const f4 v = ld_stream(reinterpret_cast<const f4*>(x + off));
    st_stream(reinterpret_cast<f4*>(y + off), ((v - s.pivot) - s.mean_d) * A + B);
}

// Normalize pass, scalar path (any alignment or slice length).
__global__ __launch_bounds__(kBlock) void split_apply_kernel(SplitGeom g, const float* x, float* y,
                                                             const GroupStat* stats,
                                                             const float* gamma,
                                                             const float* beta, float out_scale)
{
    const int64_t wg = blockIdx.x;
    const int64_t slice = wg / g.chunks;
    const int64_t ch = wg - slice * g.chunks;
    const int64_t c = slice % g.C;
    const GroupStat s = stats[group_of(g, slice)];
    const float A = s.rstd * (gamma ? gamma[c] : 1.f) * out_scale;
    const float B = (beta ? beta[c] : 0.f) * out_scale;
    const float K = s.pivot, md = s.mean_d;
    const int64_t start = ch * g.chunk;
    const int64_t len = chunk_len(g, ch);
    const int64_t off = slice * g.S + start;
    for (int64_t i = threadIdx.x; i < len; i += kBlock)
        st_stream1(y + off + i, ((ld_stream1(x + off + i) - K) - md) * A + B);
}

}  // namespace

SplitGeom split_geometry(int64_t N, int64_t C, int64_t S, bool batch, bool vec)
{
    SplitGeom g;
    g.S = S;
    g.slices = N * C;
    g.C = C;
    g.batch = batch;
    g.vec = vec;
    // Aim for >= ~2048 workgroups in flight, with chunks of at least 4096 elements and a
    // multiple of 4 * 256 so every chunk starts 16-byte aligned.
    const int64_t sl = g.slices > 0 ? g.slices : 1;  // an empty batch still gets a valid shape
    const int64_t want_chunks = (2048 + sl - 1) / sl;
    int64_t chunk = (S + want_chunks - 1) / want_chunks;
    chunk = (chunk + 1023) / 1024 * 1024;
    if (chunk < 4096) chunk = 4096;
    const int64_t s_up = (S + 1023) / 1024 * 1024;
    if (chunk > s_up) chunk = s_up;
    g.chunk = chunk;
    g.chunks = (S + chunk - 1) / chunk;
    return g;
}

namespace {
// The flat variants: slices off 16-byte boundaries in a 16-byte aligned tensor whose element
// count fits the apply step's 32-bit indexing.
bool split_flat(const SplitGeom& g, const void* x, const void* y)
{
    const int64_t T = g.slices * g.S;
    return !g.vec && T > 0 && T <= 0xFFFFFFF0LL && (uintptr_t)x % 16 == 0 &&
           (y == nullptr || (uintptr_t)y % 16 == 0);
}

template <bool FINAL>
void launch_partial(const SplitGeom& g, const float* x, const float* pre_mul, float2* partials,
                    float eps, GroupStat* stats, float* save_mean, float* save_invstd,
                    hipStream_t stream, bool cached)
{
    if (split_flat(g, x, nullptr)) {
        const int64_t units = g.slices * g.chunks;
        // the narrowest group whose one pass (16 values a lane) covers a unit's blocks
        const int64_t ulen = g.chunk < g.S ? g.chunk : g.S;
        int lanes = 4;
        while (lanes < kWave && 16 * lanes < ulen + 6) lanes *= 2;
        const int64_t per = kBlock / lanes;
        const dim3 gd((unsigned)((units + per - 1) / per)), bd(kBlock);
#define NR_PFLAT(L)                                                                                \
    if (lanes == L) {                                                                              \
        if (cached)                                                                                \
            split_partial_flat_kernel<true, FINAL, L><<<gd, bd, 0, stream>>>(                      \
                g, x, pre_mul, partials, eps, stats, save_mean, save_invstd, units);               \
        else                                                                                       \
            split_partial_flat_kernel<false, FINAL, L><<<gd, bd, 0, stream>>>(                     \
                g, x, pre_mul, partials, eps, stats, save_mean, save_invstd, units);               \
        return;                                                                                    \
    }
        NR_PFLAT(4)
        NR_PFLAT(8)
        NR_PFLAT(16)
        NR_PFLAT(32)
        NR_PFLAT(64)
#undef NR_PFLAT
        return;
    }
    const int64_t grid = g.slices * g.chunks;
    const dim3 gd((unsigned)grid), bd(kBlock);
    if (g.vec && cached)
        split_partial_kernel<true, true, FINAL><<<gd, bd, 0, stream>>>(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd);
    else if (g.vec)
        split_partial_kernel<true, false, FINAL><<<gd, bd, 0, stream>>>(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd);
    else if (cached)
        split_partial_kernel<false, true, FINAL><<<gd, bd, 0, stream>>>(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd);
    else
        split_partial_kernel<false, false, FINAL><<<gd, bd, 0, stream>>>(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd);
}

hipError_t launch_split_merge(const SplitGeom& g, const float* x, const float* pre_mul,
                              const float2* partials, float eps, GroupStat* stats,
                              float* save_mean, float* save_invstd, RunningStats run,
                              hipStream_t stream)
{
    const int64_t groups = g.batch ? g.C : g.slices;
    split_merge_kernel<<<dim3((unsigned)groups), dim3(kWave), 0, stream>>>(
        g, x, pre_mul, partials, eps, stats, save_mean, save_invstd, run);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_split_stats(const SplitGeom& g, const float* x, const float* pre_mul,
                              float2* partials, float eps, GroupStat* stats, float* save_mean,
                              float* save_invstd, RunningStats run, hipStream_t stream, bool cached)
{
    if (!g.batch && g.chunks == 1) {  // every group is one chunk: no merge step
        launch_partial<true>(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd, stream, cached);
        return hipGetLastError();
    }
    launch_partial<false>(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd, stream, cached);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_merge(g, x, pre_mul, partials, eps, stats, save_mean, save_invstd, run, stream);
}

hipError_t launch_split_apply(const SplitGeom& g, const float* x, float* y,
                              const GroupStat* stats, const float* gamma, const float* beta,
                              float out_scale, hipStream_t stream)
{
    if (split_flat(g, x, y)) {
        const int64_t nblocks = (g.slices * g.S + 3) / 4;
        split_apply_flat_kernel<<<dim3((unsigned)((nblocks + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream>>>(
            g, x, y, stats, gamma, beta, out_scale, nblocks);
        return hipGetLastError();
    }
    const int64_t subs = (g.S + 4 * kBlock - 1) / (4 * kBlock);
    const int64_t total = g.slices * subs;
    if (g.vec && total <= 0x7fffffffLL) {
        split_apply_vec_kernel<<<dim3((unsigned)total), dim3(kBlock), 0, stream>>>(
            g, x, y, stats, gamma, beta, out_scale, subs, total);
    } else {
        const int64_t grid = g.slices * g.chunks;
        split_apply_kernel<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(g, x, y, stats, gamma, beta, out_scale);
    }
    return hipGetLastError();
}

}  // namespace nr
