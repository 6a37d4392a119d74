// channels_last.hip -- the normalize -> epilogue chain over a channels-last conv output, gfx950.
//
// With c stored [N, SP, C] (C contiguous), the max over channels of the IN3d model (IN3d page,
// its step list and its note that a channels-last layout makes that max contiguous) reads one
// short contiguous run per position, while a statistics group -- (n, k) for instance norm,
// k for batch norm (BN page, opening analysis) -- becomes a column C apart.
//
//   cl_partial_kernel  one workgroup per (chunk of positions, n): thread t owns channel t % C
//                      and every (256 / C)-th position of the chunk, so each load instruction
//                      of the workgroup reads 256 consecutive floats; per thread pivot-shifted
//                      two-pass statistics over batches of 8 values, merged in position order,
//                      then the 256 / C threads of a channel merged in fixed order in LDS.
//                      Writes (count, mean - pivot, M2) per (n, chunk, k).
//   cl_merge_kernel    one wave per group, fixed-order merge of its partials; finalize (biased
//                      variance, rsqrt), optional running-statistics update.
//   cl_apply_kernel    one thread per position: per-channel coefficients staged in LDS, the C
//                      values of the position read as float4 runs, normalize, affine, scale,
//                      clamp, post-multiply, then either the max over channels or the C
//                      results written back (in place allowed).
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
        partials[(n * g.chunks + ch) * g.C + t] = make_float4(r.n, r.mean, r.m2, 0.f);
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
    Stat st = stat_empty();
    for (int64_t q = lane; q < total; q += kWave) {
        const float4 p = partials[((n0 + q / g.chunks) * g.chunks + q % g.chunks) * g.C + k];
        st = chan_merge(st, Stat{p.x, p.y, p.z});
    }
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

template <bool VEC>
__global__ __launch_bounds__(kClBlock) void cl_apply_kernel(ChainArgs a)
{
    extern __shared__ float coef_raw[];  // [C] ClCoef
    ClCoef* coef = reinterpret_cast<ClCoef*>(coef_raw);
    const int64_t n = blockIdx.y;
    const int C = (int)a.Cout;
    for (int k = threadIdx.x; k < C; k += kClBlock) {
        const GroupStat s = a.stats[a.batch ? k : n * a.Cout + k];
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
    const int64_t i = (int64_t)blockIdx.x * kClBlock + threadIdx.x;  // position in batch item n
    if (i >= a.SP) return;
    const float* cp = a.c + (n * a.SP + i) * a.Cout;
    float* op = a.out + (n * a.SP + i) * a.Cout;
    float mx = -INFINITY;
    auto one = [&](int k, float v) {
        const ClCoef q = coef[k];
        float z = (fmaf(v, q.pm, -q.pivot) - q.mean_d) * q.A + q.B;
        if (a.clamp) z = fminf(fmaxf(z, a.lo), a.hi);
        return z * q.post;
    };
    if (VEC) {
        for (int k = 0; k < C; k += 4) {
            const f4 v = *reinterpret_cast<const f4*>(cp + k);
            f4 z;
            z.x = one(k, v.x);
            z.y = one(k + 1, v.y);
            z.z = one(k + 2, v.z);
            z.w = one(k + 3, v.w);
            if (a.reduce_max_c)
                mx = fmaxf(mx, fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w)));
            else
                *reinterpret_cast<f4*>(op + k) = z;
        }
    } else {
        for (int k = 0; k < C; ++k) {
            const float z = one(k, cp[k]);
            if (a.reduce_max_c)
                mx = fmaxf(mx, z);
            else
                op[k] = z;
        }
    }
    if (a.reduce_max_c) a.out[n * a.SP + i] = mx;
}

// C / 4 = TPP lanes per position (C a multiple of 4, TPP a power of two <= 64): lane j of a
// position handles channels 4j..4j+3 with one 16-byte load, so each load instruction of a wave
// reads 1 KiB contiguously; the max over channels then finishes with log2(TPP) shuffles
// (lower lanes first). Coefficients staged in LDS as in cl_apply_kernel.
__global__ __launch_bounds__(kClBlock) void cl_apply_lanes_kernel(ChainArgs a, int tpp)
{
    extern __shared__ float coef_raw[];  // [C] ClCoef
    ClCoef* coef = reinterpret_cast<ClCoef*>(coef_raw);
    const int64_t n = blockIdx.y;
    const int C = (int)a.Cout;
    for (int k = threadIdx.x; k < C; k += kClBlock) {
        const GroupStat s = a.stats[a.batch ? k : n * a.Cout + k];
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
    const int per_block = kClBlock / tpp;
    const int j = threadIdx.x % tpp;
    const int64_t i = (int64_t)blockIdx.x * per_block + threadIdx.x / tpp;  // position
    const bool live = i < a.SP;
    f4 z = f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (live) {
        const f4 v = *reinterpret_cast<const f4*>(a.c + (n * a.SP + i) * a.Cout + 4 * j);
        auto one = [&](int k, float x) {
            const ClCoef q = coef[k];
            float r = (fmaf(x, q.pm, -q.pivot) - q.mean_d) * q.A + q.B;
            if (a.clamp) r = fminf(fmaxf(r, a.lo), a.hi);
            return r * q.post;
        };
        z.x = one(4 * j, v.x);
        z.y = one(4 * j + 1, v.y);
        z.z = one(4 * j + 2, v.z);
        z.w = one(4 * j + 3, v.w);
        if (!a.reduce_max_c) *reinterpret_cast<f4*>(a.out + (n * a.SP + i) * a.Cout + 4 * j) = z;
    }
    if (a.reduce_max_c) {
        float m = fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w));
        const int lane = threadIdx.x & (kWave - 1);
        for (int off = 1; off < tpp; off <<= 1) {  // tpp divides 64: positions never straddle waves
            const float o = __shfl_xor(m, off);
            m = (lane & off) ? fmaxf(o, m) : fmaxf(m, o);
        }
        if (live && j == 0) a.out[n * a.SP + i] = m;
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

hipError_t launch_cl_stats(const ClGeom& g, const float* c, const float* pre_mul, float4* partials,
                           float eps, GroupStat* stats, RunningStats run, hipStream_t stream)
{
    if (g.C > kClBlock) return hipErrorInvalidValue;
    cl_partial_kernel<<<dim3((unsigned)g.chunks, (unsigned)g.N), dim3(kClBlock), 0, stream>>>(
        g, c, pre_mul, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t groups = g.batch ? g.C : g.N * g.C;
    cl_merge_kernel<<<dim3((unsigned)groups), dim3(kWave), 0, stream>>>(g, c, pre_mul, partials, eps,
                                                                         stats, run);
    return hipGetLastError();
}

hipError_t launch_cl_apply(const ChainArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.SP + kClBlock - 1) / kClBlock), (unsigned)a.N);
    const size_t lds = (size_t)a.Cout * sizeof(ClCoef);
    const bool vec = a.Cout % 4 == 0 && (uintptr_t)a.c % 16 == 0 &&
                     (a.reduce_max_c || (uintptr_t)a.out % 16 == 0);
    const int64_t tpp = a.Cout / 4;
    if (vec && tpp <= kWave && (tpp & (tpp - 1)) == 0) {
        const int64_t per_block = kClBlock / tpp;
        const dim3 g2((unsigned)((a.SP + per_block - 1) / per_block), (unsigned)a.N);
        cl_apply_lanes_kernel<<<g2, dim3(kClBlock), lds, stream>>>(a, (int)tpp);
        return hipGetLastError();
    }
    if (vec)
        cl_apply_kernel<true><<<grid, dim3(kClBlock), lds, stream>>>(a);
    else
        cl_apply_kernel<false><<<grid, dim3(kClBlock), lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace nr
