// channels_last.hip -- the normalize -> epilogue chain over a channels-last conv output, gfx950.
//
// With c stored [N, SP, C] (C contiguous), the max over channels of the IN3d model (IN3d page,
// its step list and its note that a channels-last layout makes that max contiguous) reads one
// short contiguous run per position, while a statistics group -- (n, k) for instance norm,
// k for batch norm (BN page, opening analysis) -- becomes a column C apart.
//
//   cl_partial_lanes_kernel  one workgroup per (chunk of positions, n), C / 4 lanes per
//                      position, each reading 4 channels with one 16-byte load (so a load
//                      instruction of a wave reads 1 KiB contiguously); per lane and channel
//                      pivot-shifted two-pass statistics over batches of 8 positions, merged in
//                      position order, then across the lanes of a channel by a wave butterfly
//                      and across the waves in order. cl_partial_kernel does the same with
//                      one channel per thread for other C. Both write
//                      (count, mean - pivot, M2, pivot) per (n, chunk, k).
//   cl_merge_kernel    batch norm: one wave per channel, fixed-order merge of its partials over
//                      every batch item; finalize (biased variance, rsqrt), running statistics.
//   cl_apply_lanes_kernel  C / 4 lanes per position as above, 8 positions per thread, the
//                      coefficients staged in LDS. For instance norm each workgroup merges the
//                      partials of its batch item itself (chunk lanes, then a butterfly, in a
//                      fixed order), so no merge launch runs; the loads this needs go out before
//                      the data loads, and the merge overlaps them. Normalize, affine, scale,
//                      clamp, post-multiply, then the max over channels (through LDS, written as
//                      full-wave runs) or the C results written back (in place allowed).
//                      cl_apply_kernel: one thread per position, for other C or alignments.
#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

constexpr int kClBlock = 256;
constexpr int kClBatch = 8;

// Pivot of a group: its first value (position 0 of batch item 0 for a batch group, of item n
// for an instance group), times the pre-multiplier.
__device__ __forceinline__ float cl_pivot(const ClGeom& g, const float* c, int64_t n, int64_t k,
                                          float pm)
{
    return c[(g.batch ? 0 : n * g.SP) * g.C + k] * pm;
}

__global__ __launch_bounds__(kClBlock) void cl_partial_kernel(ClGeom g, const float* __restrict__ c,
                                                              const float* __restrict__ pre_mul,
                                                              float4* __restrict__ partials)
{
    __shared__ Stat part[kClBlock];
    const int C = (int)g.C;
    const int P = kClBlock / C;  // positions read side by side (C <= 256)
    const int t = threadIdx.x;
    const int k = t % C, pl = t / C;
    const int64_t n = blockIdx.y, ch = blockIdx.x;
    const int64_t p0 = ch * g.chunk;
    const int64_t p1 = min(p0 + g.chunk, g.SP);
    Stat st = stat_empty();
    if (pl < P) {
        const float pm = pre_mul ? pre_mul[k] : 1.f;
        const float K = cl_pivot(g, c, n, k, pm);
        const float* cp = c + n * g.SP * g.C + k;
        for (int64_t p = p0 + pl; p < p1; p += kClBatch * P) {
            float d[kClBatch];
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < kClBatch; ++j) {
                const int64_t pp = p + (int64_t)j * P;
                const bool v = pp < p1;  // the valid values form a prefix of the batch
                d[j] = v ? fmaf(cp[pp * g.C], pm, -K) : 0.f;
                cnt += v;
            }
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < kClBatch; ++j) s += d[j];
            const float mean = s / (float)cnt;
            float m2 = 0.f;
#pragma unroll
            for (int j = 0; j < kClBatch; ++j)
                if (j < cnt) m2 = fmaf(d[j] - mean, d[j] - mean, m2);
            st = chan_merge(st, Stat{(float)cnt, mean, m2});
        }
    }
    part[t] = st;
    __syncthreads();
    if (t < C) {
        Stat r = part[t];
        for (int j = 1; j < P; ++j) r = chan_merge(r, part[j * C + t]);
        const float pmt = pre_mul ? pre_mul[t] : 1.f;
        partials[(n * g.chunks + ch) * g.C + t] =
            make_float4(r.n, r.mean, r.m2, cl_pivot(g, c, n, t, pmt));
    }
}

// C / 4 = tpp lanes per position (C a multiple of 4, tpp a power of two <= 64): lane j of a
// position reads channels 4j..4j+3 with one 16-byte load, so each load instruction of a wave
// reads 1 KiB contiguously. Per lane and channel the same batch statistics as
// cl_partial_kernel, over the same chunk of positions; the lanes of a wave that hold the same
// channels are merged by a butterfly (lower lanes first), then the waves in order.
__global__ __launch_bounds__(kClBlock) void cl_partial_lanes_kernel(ClGeom g,
                                                                    const float* __restrict__ c,
                                                                    const float* __restrict__ pre_mul,
                                                                    float4* __restrict__ partials,
                                                                    int tpp)
{
    __shared__ Stat part[kClBlock / kWave][kClBlock];  // [wave][channel], C <= 256
    const int t = threadIdx.x;
    const int j = t % tpp, pl = t / tpp;
    const int P = kClBlock / tpp;  // positions read side by side
    const int64_t n = blockIdx.y, ch = blockIdx.x;
    const int64_t p0 = ch * g.chunk;
    const int64_t p1 = min(p0 + g.chunk, g.SP);
    float pm[4], K[4];
    Stat st[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        pm[q] = pre_mul ? pre_mul[4 * j + q] : 1.f;
        K[q] = cl_pivot(g, c, n, 4 * j + q, pm[q]);
        st[q] = stat_empty();
    }
    const float* cp = c + n * g.SP * g.C + 4 * j;
    for (int64_t p = p0 + pl; p < p1; p += kClBatch * P) {
        // the valid positions of the batch form a prefix of it
        const int cnt = (int)min<int64_t>(kClBatch, (p1 - p + P - 1) / P);
        f4 v[kClBatch];
#pragma unroll
        for (int b = 0; b < kClBatch; ++b)
            v[b] = b < cnt ? *reinterpret_cast<const f4*>(cp + (p + (int64_t)b * P) * g.C)
                           : f4{0.f, 0.f, 0.f, 0.f};
        const float inv = 1.f / (float)cnt;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float d[kClBatch];
            float s = 0.f;
#pragma unroll
            for (int b = 0; b < kClBatch; ++b) {
                d[b] = b < cnt ? fmaf(v[b][q], pm[q], -K[q]) : 0.f;
                s += d[b];
            }
            const float mean = s * inv;
            float m2 = 0.f;
#pragma unroll
            for (int b = 0; b < kClBatch; ++b)
                if (b < cnt) m2 = fmaf(d[b] - mean, d[b] - mean, m2);
            st[q] = chan_merge(st[q], Stat{(float)cnt, mean, m2});
        }
    }
    const int lane = t & (kWave - 1);
    for (int off = tpp; off < kWave; off <<= 1) {  // lanes lane ^ off hold the same channels
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            Stat o;
            o.n = __shfl_xor(st[q].n, off);
            o.mean = __shfl_xor(st[q].mean, off);
            o.m2 = __shfl_xor(st[q].m2, off);
            st[q] = upper ? chan_merge(o, st[q]) : chan_merge(st[q], o);
        }
    }
    const int wave = t / kWave;
    if (lane < tpp) {
#pragma unroll
        for (int q = 0; q < 4; ++q) part[wave][4 * lane + q] = st[q];
    }
    __syncthreads();
    if (t < (int)g.C) {
        Stat r = part[0][t];
        for (int w = 1; w < kClBlock / kWave; ++w) r = chan_merge(r, part[w][t]);
        const float pmt = pre_mul ? pre_mul[t] : 1.f;
        partials[(n * g.chunks + ch) * g.C + t] =
            make_float4(r.n, r.mean, r.m2, cl_pivot(g, c, n, t, pmt));
    }
}

__global__ __launch_bounds__(kWave) void cl_merge_kernel(ClGeom g, const float* __restrict__ c,
                                                         const float* __restrict__ pre_mul,
                                                         const float4* __restrict__ partials,
                                                         float eps, GroupStat* __restrict__ stats,
                                                         RunningStats run)
{
    const int64_t grp = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t k = g.batch ? grp : grp % g.C;
    const int64_t n0 = g.batch ? 0 : grp / g.C;
    const int64_t members = g.batch ? g.N : 1;  // batch items merged into this group
    const int64_t total = members * g.chunks;
    Stat st = lane_strided_merge<kWave>(total, [&](int64_t q) {
        const float4 p = partials[((n0 + q / g.chunks) * g.chunks + q % g.chunks) * g.C + k];
        return Stat{p.x, p.y, p.z};
    });
    st = wave_merge<kWave>(st);
    if (lane == 0) {
        const float pm = pre_mul ? pre_mul[k] : 1.f;
        const float K = cl_pivot(g, c, n0, k, pm);
        const float rstd = rsqrtf(st.m2 / st.n + eps);
        stats[grp] = GroupStat{K, st.mean, rstd, 0.f};
        if (run.mean) {
            // BN page, opening analysis: running = (1 - m) * running + m * batch, with the
            // unbiased batch variance
            const float m = run.momentum;
            run.mean[grp] = (1.f - m) * run.mean[grp] + m * (K + st.mean);
            run.var[grp] = (1.f - m) * run.var[grp] + m * (st.m2 / (st.n - 1.f));
        }
    }
}

// Per-channel coefficients of one batch item: z = ((v * pm - pivot) - mean_d) * A + B, then
// clamp, then * post (the pivot is removed first, as in the statistics).
struct ClCoef {
    float pm, pivot, mean_d, A, B, post;
};

// Where the apply kernels take the statistics of a group. Batch norm: the merged statistics
// (its merge also updates the running statistics). Instance norm: the partials of batch item
// n, merged by each apply workgroup itself, so no merge launch runs; every workgroup of item n
// merges the same partials in the same order and sees the same values.
struct ClSrc {
    ClGeom g;
    const float4* partials;  // instance norm: [N, chunks, C]; batch norm: NULL
    float eps;
};

// Stages the coefficients of batch item n into coef (one-thread-per-position kernel); every
// thread of the workgroup calls it (it holds barriers) and the staged values are visible when
// it returns. For instance norm the R = kClBlock / C threads of a channel first merge its
// partials chunk-strided (thread r of the channel takes chunks r, r + R, ...), then one thread
// merges their results in order of r. The pivot travels in the partials: with the output
// written in place, position 0 of c may already hold its result.
__device__ __forceinline__ void cl_stage_coef(const ChainArgs& a, const ClSrc& src, int64_t n,
                                              ClCoef* coef, Stat* red /* [kClBlock] */)
{
    const int C = (int)a.Cout;  // <= kClBlock
    const int t = threadIdx.x;
    const int R = kClBlock / C;
    if (src.partials) {
        const int k = t % C, r = t / C;
        if (r < R) {
            const float4* pp = src.partials + n * src.g.chunks * C + k;
            Stat st = stat_empty();
            for (int64_t q = r; q < src.g.chunks; q += R) {
                const float4 v = pp[q * C];
                st = chan_merge(st, Stat{v.x, v.y, v.z});
            }
            red[t] = st;
        }
        __syncthreads();
    }
    if (t < C) {
        const int k = t;
        GroupStat s;
        if (src.partials) {
            Stat st = red[k];
            for (int r = 1; r < R; ++r) st = chan_merge(st, red[r * C + k]);
            const float pivot = src.partials[n * src.g.chunks * C + k].w;
            s = GroupStat{pivot, st.mean, rsqrtf(st.m2 / st.n + src.eps), 0.f};
        } else {
            s = a.stats[a.batch ? k : n * a.Cout + k];
        }
        ClCoef q;
        q.pm = a.pre_mul ? a.pre_mul[k] : 1.f;
        q.pivot = s.pivot;
        q.mean_d = s.mean_d;
        q.A = s.rstd * (a.gamma ? a.gamma[k] : 1.f) * a.out_scale;
        q.B = (a.beta ? a.beta[k] : 0.f) * a.out_scale;
        q.post = a.post_mul ? a.post_mul[k] : 1.f;
        coef[k] = q;
    }
    __syncthreads();
}

// The lanes kernel stages in two halves around its data loads: cl_stage_issue loads what the
// coefficients need (the partials of each chunk lane and the pivot for instance norm, or the
// merged statistics for batch norm, and the per-channel parameters) before the data loads are
// issued, so that cl_stage_finish, which waits only for these, overlaps the merge with the data
// in flight. Thread t serves channel t / R and chunk lane r = t % R (R = kClBlock / C, a power
// of two <= 64); the chunk lanes then merge by a butterfly across the R adjacent lanes (lower
// lanes first), a fixed order. Every load here is unconditional (indexes clamped): a load under
// a branch is waited for at the branch's end.
struct ClStage {
    float4 p0;                  // instance norm: partial of chunk min(r, chunks - 1)
    Stat extra;                 // instance norm: chunks r + R, r + 2R, ... merged in order
    float pivot, mean_d, rstd;  // the pivot; batch norm: the merged statistics
    float pm, gm, bt, qm;
};

template <bool INST>
__device__ __forceinline__ ClStage cl_stage_issue(const ChainArgs& a, const ClSrc& src, int64_t n)
{
    const int C = (int)a.Cout;
    const int R = kClBlock / C;
    const int k = threadIdx.x / R, r = threadIdx.x % R;
    ClStage S;
    S.pm = *(a.pre_mul ? a.pre_mul + k : &kParamOne);
    S.gm = *(a.gamma ? a.gamma + k : &kParamOne);
    S.bt = *(a.beta ? a.beta + k : &kParamZero);
    S.qm = *(a.post_mul ? a.post_mul + k : &kParamOne);
    if (INST) {
        const float4* pp = src.partials + n * src.g.chunks * C + k;
        // chunks r + R, r + 2R, ... (only when chunks > R), 8 loads at a time
        S.extra = src.g.chunks > R ? lane_strided_merge_by(src.g.chunks - R, R, [&](int64_t q) {
            const float4 v = pp[(q + R) * C];
            return Stat{v.x, v.y, v.z};
        }) : stat_empty();
        S.p0 = pp[min<int64_t>(r, src.g.chunks - 1) * C];  // chunks >= 1
        S.pivot = pp[0].w;
        S.mean_d = S.rstd = 0.f;
    } else {
        const GroupStat g = a.stats[a.batch ? k : n * a.Cout + k];
        S.pivot = g.pivot;
        S.mean_d = g.mean_d;
        S.rstd = g.rstd;
    }
    return S;
}

template <bool INST>
__device__ __forceinline__ void cl_stage_finish(const ChainArgs& a, const ClSrc& src,
                                                const ClStage& S, ClCoef* coef)
{
    const int C = (int)a.Cout;
    const int R = kClBlock / C;
    const int k = threadIdx.x / R, r = threadIdx.x % R;
    float mean_d = S.mean_d, rstd = S.rstd;
    if (INST) {
        Stat st = r < src.g.chunks ? Stat{S.p0.x, S.p0.y, S.p0.z} : stat_empty();
        st = chan_merge(st, S.extra);
        const int lane = threadIdx.x & (kWave - 1);
        for (int off = 1; off < R; off <<= 1) {
            Stat o;
            o.n = __shfl_xor(st.n, off);
            o.mean = __shfl_xor(st.mean, off);
            o.m2 = __shfl_xor(st.m2, off);
            st = (lane & off) ? chan_merge(o, st) : chan_merge(st, o);
        }
        mean_d = st.mean;
        rstd = rsqrtf(st.m2 / st.n + src.eps);
    }
    if (r == 0) {
        ClCoef q;
        q.pm = S.pm;
        q.pivot = S.pivot;
        q.mean_d = mean_d;
        q.A = rstd * S.gm * a.out_scale;
        q.B = S.bt * a.out_scale;
        q.post = S.qm;
        coef[k] = q;
    }
    __syncthreads();
}

__device__ __forceinline__ float cl_value(const ChainArgs& a, const ClCoef& q, float v)
{
    float z = (fmaf(v, q.pm, -q.pivot) - q.mean_d) * q.A + q.B;
    if (a.clamp) z = fminf(fmaxf(z, a.lo), a.hi);
    return z * q.post;
}

template <bool VEC>
__global__ __launch_bounds__(kClBlock) void cl_apply_kernel(ChainArgs a, ClSrc src)
{
    extern __shared__ float coef_raw[];  // [C] ClCoef
    __shared__ Stat red[kClBlock];
    ClCoef* coef = reinterpret_cast<ClCoef*>(coef_raw);
    const int64_t n = blockIdx.y;
    const int C = (int)a.Cout;
    cl_stage_coef(a, src, n, coef, red);
    const int64_t i = (int64_t)blockIdx.x * kClBlock + threadIdx.x;  // position in batch item n
    if (i >= a.SP) return;
    const float* cp = a.c + (n * a.SP + i) * a.Cout;
    float* op = a.out + (n * a.SP + i) * a.Cout;
    float mx = -INFINITY;
    if (VEC) {
        for (int k = 0; k < C; k += 4) {
            const f4 v = *reinterpret_cast<const f4*>(cp + k);
            f4 z;
            z.x = cl_value(a, coef[k], v.x);
            z.y = cl_value(a, coef[k + 1], v.y);
            z.z = cl_value(a, coef[k + 2], v.z);
            z.w = cl_value(a, coef[k + 3], v.w);
            if (a.reduce_max_c)
                mx = fmaxf(mx, fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w)));
            else
                *reinterpret_cast<f4*>(op + k) = z;
        }
    } else {
        for (int k = 0; k < C; ++k) {
            const float z = cl_value(a, coef[k], cp[k]);
            if (a.reduce_max_c)
                mx = fmaxf(mx, z);
            else
                op[k] = z;
        }
    }
    if (a.reduce_max_c) a.out[n * a.SP + i] = mx;
}

// C / 4 = tpp lanes per position (C a multiple of 4, tpp a power of two <= 64): lane j of a
// position handles channels 4j..4j+3 with one 16-byte load, so each load instruction of a wave
// reads 1 KiB contiguously; U positions per thread, kClBlock / tpp apart, loaded together. The
// max over channels finishes with log2(tpp) shuffles (lower lanes first) and leaves through LDS
// as full-wave runs of consecutive positions.
template <int U, bool INST, bool MAXC>
__global__ __launch_bounds__(kClBlock) void cl_apply_lanes_kernel(ChainArgs a, ClSrc src, int tpp)
{
    extern __shared__ float coef_raw[];  // [C] ClCoef
    __shared__ float mx[MAXC ? kClBlock * U : 1];  // the workgroup's maxima, in position order
    ClCoef* coef = reinterpret_cast<ClCoef*>(coef_raw);
    const int64_t n = blockIdx.y;
    const int per_load = kClBlock / tpp;  // positions per load instruction of the workgroup
    const int j = threadIdx.x % tpp;
    const int64_t base = (int64_t)blockIdx.x * per_load * U;
    const int64_t i0 = base + threadIdx.x / tpp;
    const float* cp = a.c + n * a.SP * a.Cout + 4 * j;
    const ClStage S = cl_stage_issue<INST>(a, src, n);  // R = 64 / tpp: a power of two <= 64
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // positions past the end load the last one (unused)
        const int64_t i = min(i0 + (int64_t)u * per_load, a.SP - 1);
        v[u] = *reinterpret_cast<const f4*>(cp + i * a.Cout);
    }
    cl_stage_finish<INST>(a, src, S, coef);
    const ClCoef q0 = coef[4 * j], q1 = coef[4 * j + 1], q2 = coef[4 * j + 2], q3 = coef[4 * j + 3];
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * per_load;
        f4 z;
        z.x = cl_value(a, q0, v[u].x);
        z.y = cl_value(a, q1, v[u].y);
        z.z = cl_value(a, q2, v[u].z);
        z.w = cl_value(a, q3, v[u].w);
        if (MAXC) {
            float m = fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w));
            for (int off = 1; off < tpp; off <<= 1) {  // tpp divides 64: positions never straddle waves
                const float o = __shfl_xor(m, off);
                m = (lane & off) ? fmaxf(o, m) : fmaxf(m, o);
            }
            if (j == 0) mx[u * per_load + threadIdx.x / tpp] = m;
        } else if (i < a.SP) {
            st_stream(reinterpret_cast<f4*>(a.out + (n * a.SP + i) * a.Cout + 4 * j), z);
        }
    }
    if (MAXC) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < per_load * U; idx += kClBlock)
            if (base + idx < a.SP) st_stream1(a.out + n * a.SP + base + idx, mx[idx]);
    }
}

}  // namespace

ClGeom cl_geometry(int64_t N, int64_t C, int64_t SP, bool batch)
{
    ClGeom g;
    g.N = N;
    g.C = C;
    g.SP = SP;
    g.batch = batch;
    const int64_t P = C <= kClBlock ? kClBlock / C : 1;
    g.chunk = 8 * kClBatch * P;  // 64 values per thread
    g.chunks = SP > 0 ? (SP + g.chunk - 1) / g.chunk : 0;
    return g;
}

size_t cl_partials_bytes(const ClGeom& g) { return (size_t)(g.N * g.chunks * g.C) * sizeof(float4); }

namespace {
// 16-byte loads of 4 channels per lane: C a multiple of 4 with C / 4 a power of two (<= 64
// since C <= 256), c 16-byte aligned.
bool cl_lanes(int64_t C, const void* c)
{
    const int64_t tpp = C / 4;
    return C % 4 == 0 && tpp >= 1 && (tpp & (tpp - 1)) == 0 && (uintptr_t)c % 16 == 0;
}

constexpr int kClApplyU = 8;  // positions per thread of cl_apply_lanes_kernel
}  // namespace

hipError_t launch_cl_stats(const ClGeom& g, const float* c, const float* pre_mul, float4* partials,
                           float eps, GroupStat* stats, RunningStats run, hipStream_t stream)
{
    if (g.C > kClBlock) return hipErrorInvalidValue;
    const dim3 grid((unsigned)g.chunks, (unsigned)g.N);
    if (cl_lanes(g.C, c))
        cl_partial_lanes_kernel<<<grid, dim3(kClBlock), 0, stream>>>(g, c, pre_mul, partials,
                                                                      (int)(g.C / 4));
    else
        cl_partial_kernel<<<grid, dim3(kClBlock), 0, stream>>>(g, c, pre_mul, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !g.batch) return e;  // instance norm: the apply kernel merges
    cl_merge_kernel<<<dim3((unsigned)g.C), dim3(kWave), 0, stream>>>(g, c, pre_mul, partials, eps,
                                                                      stats, run);
    return hipGetLastError();
}

hipError_t launch_cl_apply(const ChainArgs& a, const ClGeom& g, const float4* partials, float eps,
                           hipStream_t stream)
{
    const ClSrc src{g, a.batch ? nullptr : partials, eps};
    const size_t lds = (size_t)a.Cout * sizeof(ClCoef);
    const bool vec = a.Cout % 4 == 0 && (uintptr_t)a.c % 16 == 0 &&
                     (a.reduce_max_c || (uintptr_t)a.out % 16 == 0);
    if (vec && cl_lanes(a.Cout, a.c)) {
        const int tpp = (int)(a.Cout / 4);
        const int64_t per_wg = (int64_t)(kClBlock / tpp) * kClApplyU;
        const dim3 grid((unsigned)((a.SP + per_wg - 1) / per_wg), (unsigned)a.N);
        const dim3 block(kClBlock);
        const bool inst = src.partials != nullptr, maxc = a.reduce_max_c != 0;
        if (inst && maxc)
            cl_apply_lanes_kernel<kClApplyU, true, true><<<grid, block, lds, stream>>>(a, src, tpp);
        else if (inst)
            cl_apply_lanes_kernel<kClApplyU, true, false><<<grid, block, lds, stream>>>(a, src, tpp);
        else if (maxc)
            cl_apply_lanes_kernel<kClApplyU, false, true><<<grid, block, lds, stream>>>(a, src, tpp);
        else
            cl_apply_lanes_kernel<kClApplyU, false, false><<<grid, block, lds, stream>>>(a, src, tpp);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((a.SP + kClBlock - 1) / kClBlock), (unsigned)a.N);
    if (vec)
        cl_apply_kernel<true><<<grid, dim3(kClBlock), lds, stream>>>(a, src);
    else
        cl_apply_kernel<false><<<grid, dim3(kClBlock), lds, stream>>>(a, src);
    return hipGetLastError();
}

}  // namespace nr
