// inorm_resident.hip -- read-once instance normalization for gfx950.
//
// Operation: IN2d page (task l1_p34), statement of the op: per (n, c) slice, mean and biased
// variance over the spatial extent, y = (x - mean)/sqrt(var + eps) (* gamma[c] + beta[c]).
//
// Design (MI355X-first; the page's own kernel reads each slice twice -- a Welford pass and a
// normalize pass -- which caps a bandwidth-bound kernel at two thirds of the HBM roofline):
//   * A slice is split into P parts (1 <= P <= 32). One workgroup owns a part and keeps it in
//     VGPRs from load to store, so x crosses HBM exactly once and y once.
//   * Per thread: 16-byte non-temporal loads; statistics of its own values by the two-pass
//     formula over registers, relative to a per-slice pivot K = x[slice][0] (removes the
//     offset before any sum: the cancellation the page's numerics discussion worries about).
//   * Wave64 butterfly merges of (count, mean, M2) and an LDS combine across waves. Parts
//     that fill their workgroup give every lane the same count, so those merges use the
//     equal-count form (no division); ragged parts use the general pairwise update.
//   * P == 1 (slices up to 64K elements): one workgroup per slice, hardware dispatch.
//   * P > 1: a persistent grid of co-resident workgroups (cooperative launch) takes units
//     (slice, part) from an atomic counter in increasing order, so fast CUs take more units
//     (a static assignment leaves the grid waiting on its slowest CU). Each workgroup holds
//     two units in two register buffers: it loads the next unit and publishes that unit's
//     statistics before it waits for the siblings of the unit it loaded before, then
//     normalizes and stores that one. The wait therefore overlaps a whole unit of memory
//     traffic instead of stalling it.
//   * Exchange: (mean, M2) of a part go out as two tagged 64-bit words with relaxed
//     agent-scope atomic stores; siblings poll them the same way. The counter and slot region
//     are zero-filled just before every launch, so a non-zero tag marks a word written by
//     this launch; every exchanged word carries its own validity tag, so no cache-wide
//     release/acquire fences are needed. The P partials are merged in part order 0..P-1 by
//     every sibling, so all parts normalize with identical statistics and the result does not
//     depend on arrival order or on which workgroup took which part.
//   * Forward progress: a workgroup takes a new unit only after its pending wait finished
//     and always publishes a unit before its next wait, so every waiting workgroup holds only
//     published units (at most two). Units are handed out in order, so only the highest slice
//     in flight can miss parts; if every workgroup waited on that slice, each would hold two
//     of its parts, which needs 2G <= P - 1 -- impossible with G >= P co-resident workgroups.
//   * Normalize from registers: y = d * (rstd * gamma) + (beta - mean_d * rstd * gamma) with
//     d = x - K, one fused multiply-add per element, 16-byte non-temporal stores.
#include <stdlib.h>

#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

// Tag of an exchange word written by the current launch (the slots start zeroed).
constexpr uint32_t kTag = 1u;

// Equal-count butterfly: every lane holds the same count; after log2(WIDTH) levels every lane
// of an aligned group of WIDTH lanes holds the group's statistics.
template <int WIDTH>
__device__ __forceinline__ Stat wave_merge_equal(Stat s)
{
#pragma unroll
    for (int off = 1; off < WIDTH; off <<= 1) {
        const float om = __shfl_xor(s.mean, off);
        const float oq = __shfl_xor(s.m2, off);
        const float d = om - s.mean;  // squared below: the sign does not matter
        s.m2 = (s.m2 + oq) + d * d * (0.5f * s.n);
        s.mean = (s.mean + om) * 0.5f;
        s.n *= 2.f;
    }
    return s;
}

// One part held in registers: VEC float4 per thread, already shifted by the pivot.
template <int BLOCK, int VEC>
struct Part {
    f4 v[VEC];

    __device__ __forceinline__ void load(const float* x, int64_t off, int nvec, bool full, float K)
    {
        const f4* xs = reinterpret_cast<const f4*>(x + off);
        const int tid = threadIdx.x;
        if (full) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) v[j] = ld_stream(xs + j * BLOCK + tid);
#pragma unroll
            for (int j = 0; j < VEC; ++j) v[j] -= K;
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int i = j * BLOCK + tid;
                v[j] = i < nvec ? ld_stream(xs + i) - K : f4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    // This thread's (count, mean, M2): two passes over its registers.
    __device__ __forceinline__ Stat thread_stat(int nvec, bool full) const
    {
        const int tid = threadIdx.x;
        int nv = VEC;
        if (!full) {
            nv = 0;
#pragma unroll
            for (int j = 0; j < VEC; ++j) nv += (j * BLOCK + tid < nvec) ? 1 : 0;
        }
        f4 s = v[0];  // invalid entries are zero, so they add nothing to the sum
#pragma unroll
        for (int j = 1; j < VEC; ++j) s += v[j];
        const float cnt = (float)(4 * nv);
        const float sum = (s.x + s.y) + (s.z + s.w);
        const float m = full ? sum * (1.0f / (float)(4 * VEC)) : (nv > 0 ? sum / cnt : 0.f);
        f4 q = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            if (full || j * BLOCK + tid < nvec) {
                const f4 e = v[j] - m;
                q += e * e;
            }
        }
        return Stat{cnt, m, (q.x + q.y) + (q.z + q.w)};
    }

    __device__ __forceinline__ void store(float* y, int64_t off, int nvec, bool full, float sc,
                                          float sh) const
    {
        f4* ys = reinterpret_cast<f4*>(y + off);
        const int tid = threadIdx.x;
        if (full) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) st_stream(ys + j * BLOCK + tid, v[j] * sc + sh);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int i = j * BLOCK + tid;
                if (i < nvec) st_stream(ys + i, v[j] * sc + sh);
            }
        }
    }
};

// Geometry of one unit (slice, part).
struct UnitGeo {
    int64_t slice, off;  // off: element offset of the part
    int part, plen, nvec;
    bool full;
};

template <int PART>
__device__ __forceinline__ UnitGeo unit_geo(const ResidentArgs& a, int64_t u)
{
    UnitGeo g;
    g.slice = u / a.P;
    g.part = (int)(u - g.slice * a.P);
    const int64_t pstart = (int64_t)g.part * PART;
    const int64_t rem = a.S - pstart;
    g.plen = rem < PART ? (int)rem : PART;
    g.nvec = g.plen >> 2;
    g.full = g.plen == PART;
    g.off = g.slice * a.S + pstart;
    return g;
}

// Statistics of a part: thread stats -> wave merge -> LDS; wave 0 then merges the waves
// (every lane of wave 0 holds the result). Contains one workgroup barrier.
template <int BLOCK, int VEC>
__device__ __forceinline__ Stat part_stats(const Part<BLOCK, VEC>& p, const UnitGeo& g, Stat* wstat)
{
    constexpr int NW = BLOCK / kWave;
    Stat st = p.thread_stat(g.nvec, g.full);
    st = g.full ? wave_merge_equal<kWave>(st) : wave_merge<kWave>(st);
    if (lane_id() == 0) wstat[threadIdx.x / kWave] = st;
    __syncthreads();
    Stat w = stat_empty();
    if (threadIdx.x < kWave) {
        w = lane_id() < NW ? wstat[lane_id()] : stat_empty();
        // lanes 0..NW-1 form one aligned group; in a full part all NW counts are equal
        w = g.full ? wave_merge_equal<NW>(w) : wave_merge<NW>(w);
    }
    return w;
}

// Final per-slice coefficients: y = d * fin[0] + fin[1].
__device__ __forceinline__ void finalize(const ResidentArgs& a, int64_t slice, int part, float K,
                                         Stat w, float* fin)
{
    const float var = w.m2 / w.n;
    const float rstd = rsqrtf(var + a.eps);
    const int64_t c = slice % a.C;
    const float g = a.gamma ? a.gamma[c] : 1.f;
    const float b = a.beta ? a.beta[c] : 0.f;
    const float sc = rstd * g;
    fin[0] = sc;
    fin[1] = fmaf(-w.mean, sc, b);
    if (part == 0 && a.save_mean) a.save_mean[slice] = K + w.mean;
    if (part == 0 && a.save_invstd) a.save_invstd[slice] = rstd;
}

// ---------------------------------------------------------------------------------------------
// P == 1: one workgroup per slice.
// ---------------------------------------------------------------------------------------------
template <int BLOCK, int VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(BLOCK, BLOCK), amdgpu_waves_per_eu(4))) void
inorm_single_kernel(ResidentArgs a)
{
    constexpr int PART = BLOCK * 4 * VEC;
    __shared__ Stat wstat[BLOCK / kWave];
    __shared__ float fin[2];
    const int64_t slice = blockIdx.x;
    const UnitGeo g = unit_geo<PART>(a, slice);
    const float K = a.x[slice * a.S];
    Part<BLOCK, VEC> p;
    p.load(a.x, g.off, g.nvec, g.full, K);
    const Stat w = part_stats<BLOCK, VEC>(p, g, wstat);
    if (threadIdx.x == 0) finalize(a, slice, 0, K, w, fin);
    __syncthreads();
    p.store(a.y, g.off, g.nvec, g.full, fin[0], fin[1]);
}

// ---------------------------------------------------------------------------------------------
// P > 1: persistent, two units per workgroup.
// ---------------------------------------------------------------------------------------------
// Publish one part's statistics (thread 0).
__device__ __forceinline__ void publish(const ResidentArgs& a, const UnitGeo& g, Stat w)
{
    if (threadIdx.x == 0) {
        unsigned long long* sl = a.slots + (size_t)g.slice * a.P * 2;
        xchg_store(sl + g.part * 2 + 0, kTag, w.mean);
        xchg_store(sl + g.part * 2 + 1, kTag, w.m2);
    }
}

// Wave 0: wait for all parts of `slice`, merge them in part order, write fin (lane 0).
template <int PART>
__device__ __forceinline__ void gather(const ResidentArgs& a, int64_t slice, int part, float K,
                                       float* fin)
{
    const int lane = lane_id();
    unsigned long long* sl = a.slots + (size_t)slice * a.P * 2;
    Stat ps = stat_empty();
    if (lane < a.P) {
        unsigned long long w0, w1;
        uint32_t spins = 0;
        for (;;) {
            w0 = xchg_load(sl + lane * 2 + 0);
            w1 = xchg_load(sl + lane * 2 + 1);
            if ((uint32_t)(w0 >> 32) == kTag && (uint32_t)(w1 >> 32) == kTag) break;
            if (++spins > kSpinLimit) {
                raise_flag(a.flags, kFlagSpinTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        const int64_t prem = a.S - (int64_t)lane * PART;
        ps.n = (float)(prem < PART ? prem : PART);
        ps.mean = __uint_as_float((uint32_t)w0);
        ps.m2 = __uint_as_float((uint32_t)w1);
    }
    const Stat w = wave_merge<kMaxParts>(ps);  // parts merged in order 0..P-1
    if (lane == 0) finalize(a, slice, part, K, w, fin);
}

template <int BLOCK, int VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(BLOCK, BLOCK), amdgpu_waves_per_eu(2))) void
inorm_pipelined_kernel(ResidentArgs a)
{
    constexpr int PART = BLOCK * 4 * VEC;
    __shared__ Stat wstat[BLOCK / kWave];
    __shared__ float fin[2];
    __shared__ uint32_t next_unit;
    const int64_t units = a.slices * a.P;

    // One pipeline step: load unit `un` into `ldp` and publish its statistics (if valid); then
    // wave 0 waits for the parts of unit `uo` held in `wtp` (if valid) and takes the next unit;
    // then `wtp` is normalized and stored. Returns the unit taken next.
    auto step = [&](Part<BLOCK, VEC>& ldp, int64_t un, float& Kn, const Part<BLOCK, VEC>& wtp,
                    int64_t uo, float Ko) -> int64_t {
        if (un < units) {
            const UnitGeo gn = unit_geo<PART>(a, un);
            Kn = a.x[gn.slice * a.S];
            ldp.load(a.x, gn.off, gn.nvec, gn.full, Kn);
            const Stat w = part_stats<BLOCK, VEC>(ldp, gn, wstat);  // contains a barrier
            publish(a, gn, w);
        }
        UnitGeo go{};
        if (uo < units) go = unit_geo<PART>(a, uo);
        if (threadIdx.x < kWave) {
            if (uo < units) gather<PART>(a, go.slice, go.part, Ko, fin);
            // after the wait, with every held unit published: take the next unit
            if (threadIdx.x == 0)
                next_unit = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const int64_t nx = next_unit;
        if (uo < units) wtp.store(a.y, go.off, go.nvec, go.full, fin[0], fin[1]);
        __syncthreads();  // fin and next_unit are rewritten by the next step
        return nx;
    };

    Part<BLOCK, VEC> A, B;
    float KA = 0.f, KB = 0.f;
    if (threadIdx.x == 0)
        next_unit = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int64_t ua = next_unit;  // unit going into A
    int64_t ub = units;      // unit held in B (none yet)
    __syncthreads();
    for (;;) {
        const int64_t n1 = step(A, ua, KA, B, ub, KB);  // load A, finish B
        if (ua >= units) break;                         // A empty, B done
        ub = n1;
        const int64_t n2 = step(B, ub, KB, A, ua, KA);  // load B, finish A
        if (ub >= units) break;                         // B empty, A done
        ua = n2;
    }
}

struct Entry {
    ResidentCfg cfg;
    const void* fn;
};

#define NR_SINGLE(B, V) \
    Entry { ResidentCfg{B, V, B * 4 * V, false}, reinterpret_cast<const void*>(&inorm_single_kernel<B, V>) }
#define NR_PIPE(B, V) \
    Entry { ResidentCfg{B, V, B * 4 * V, true}, reinterpret_cast<const void*>(&inorm_pipelined_kernel<B, V>) }

// Single-workgroup configurations ascending by part length, then the pipelined ones ascending.
const Entry kCfgs[] = {
    NR_SINGLE(256, 1),  NR_SINGLE(256, 2),  NR_SINGLE(256, 4), NR_SINGLE(256, 8),
    NR_SINGLE(256, 16), NR_SINGLE(512, 16), NR_SINGLE(1024, 16),
    NR_PIPE(256, 8),    NR_PIPE(256, 16),   NR_PIPE(512, 16),
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

const void* cfg_fn(const ResidentCfg& c)
{
    for (int i = 0; i < kNumCfgs; ++i)
        if (kCfgs[i].cfg.block == c.block && kCfgs[i].cfg.vec == c.vec &&
            kCfgs[i].cfg.pipelined == c.pipelined)
            return kCfgs[i].fn;
    return nullptr;
}

int env_int(const char* name, int dflt)
{
    const char* e = getenv(name);
    if (!e || !*e) return dflt;
    const int v = atoi(e);
    return v > 0 ? v : dflt;
}

}  // namespace

int resident_cfg_count() { return kNumCfgs; }
ResidentCfg resident_cfg(int i) { return kCfgs[i].cfg; }

int resident_max_grid(const ResidentCfg& cfg)
{
    const void* fn = cfg_fn(cfg);
    if (!fn) return 0;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, cfg.block, 0) != hipSuccess)
        return 0;
    // The pipelined kernel streams best with two workgroups per CU (more of them interleave
    // more streams into the DRAM pages and lose bandwidth); NORMRED_RESIDENT_WGS_PER_CU
    // overrides it for tuning.
    if (cfg.pipelined) {
        const int want = env_int("NORMRED_RESIDENT_WGS_PER_CU", 2);
        if (per_cu > want) per_cu = want;
    }
    return cus * per_cu;
}

hipError_t launch_resident(const ResidentCfg& cfg, const ResidentArgs& a, hipStream_t stream)
{
    const void* fn = cfg_fn(cfg);
    if (!fn) return hipErrorInvalidDeviceFunction;
    ResidentArgs args = a;
    void* params[] = {&args};
    if (!cfg.pipelined) {
        if (a.P != 1) return hipErrorInvalidValue;
        const int64_t grid = a.slices;  // validated <= 2^31 - 1 by the caller
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(cfg.block), params, 0, stream);
    }
    const int64_t units = a.slices * a.P;
    int64_t grid = resident_max_grid(cfg);
    if (grid > units) grid = units;
    if (grid < a.P) return hipErrorCooperativeLaunchTooLarge;  // the P parts must co-reside
    // counter + slots start zeroed for every launch (they carry nothing between calls)
    const hipError_t e = launch_fill_zero(a.counter, resident_ws_bytes(a.slices, a.P), stream);
    if (e != hipSuccess) return e;
    const char* coop = getenv("NORMRED_COOPERATIVE");
    if (coop && coop[0] == '0')  // same grid, regular launch (profilers)
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(cfg.block), params, 0, stream);
    return hipLaunchCooperativeKernel(fn, dim3((unsigned)grid), dim3(cfg.block), params, 0, stream);
}

}  // namespace nr
