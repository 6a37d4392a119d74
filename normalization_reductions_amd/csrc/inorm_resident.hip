// inorm_resident.hip -- read-once instance normalization for gfx950.
//
// Operation: IN2d page (task l1_p34), statement of the op: per (n, c) slice, mean and biased
// variance over the spatial extent, y = (x - mean)/sqrt(var + eps) (* gamma[c] + beta[c]).
//
// Design (MI355X-first; the page's own kernel reads each slice twice -- a Welford pass and a
// normalize pass -- which caps a bandwidth-bound kernel at two thirds of the HBM roofline):
//   * A slice is split into P parts (1 <= P <= 16). One workgroup owns one part and
//     keeps it in VGPRs from load to store, so x crosses HBM exactly once and y once.
//   * Per thread: 16-byte non-temporal loads, statistics of its own values by the two-pass
//     formula over registers, relative to a per-slice pivot K = x[slice][0] (removes the
//     offset before any sum: the cancellation the page's numerics discussion worries about).
//   * Wave64 butterfly Chan merges, then an LDS combine across the workgroup's waves.
//   * P > 1: the P workgroups of a slice are co-resident (cooperative launch of a persistent
//     grid whose size is a multiple of P; units are dealt so that the same P consecutive
//     workgroups own the P parts of a slice in every round). Each publishes (mean, M2) as two
//     tagged 64-bit words with relaxed agent-scope atomic stores and polls its siblings' words
//     the same way. The slot region is zero-filled just before the launch, so a non-zero tag
//     marks a word written by this launch; because every exchanged word carries its own
//     validity tag, no cache-wide release/acquire fences are needed. The P partials are merged
//     in part order 0..P-1 by every sibling, so all parts normalize with identical statistics
//     and the result does not depend on arrival order.
//   * Normalize from registers: y = ((x - K) - mean_d) * (rstd * gamma) + beta, 16-byte
//     non-temporal stores.
#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

// Tag of an exchange word written by the current launch (the slots start zeroed).
constexpr uint32_t kTag = 1u;

template <int BLOCK, int VEC, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(BLOCK, BLOCK),
                          amdgpu_waves_per_eu(WAVES_PER_EU))) void
inorm_resident_kernel(ResidentArgs a)
{
    constexpr int NW = BLOCK / kWave;
    constexpr int PART = BLOCK * 4 * VEC;
    static_assert(NW >= 1 && NW <= kWave, "workgroup size");

    __shared__ Stat wstat[NW];
    __shared__ float fin[3];  // mean_d, scale, shift

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wid = tid / kWave;
    const int P = a.P;
    const int64_t units = a.slices * P;

    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t slice = u / P;
        const int part = (int)(u - slice * P);
        const int64_t base = slice * a.S;
        const int64_t pstart = (int64_t)part * PART;
        const int64_t rem = a.S - pstart;
        const int plen = rem <= 0 ? 0 : (rem < PART ? (int)rem : PART);
        const int nvec = plen >> 2;

        const float K = a.x[base];  // pivot, read before any part of this slice is written
        const f4* xs = reinterpret_cast<const f4*>(a.x + base + pstart);
        f4* ys = reinterpret_cast<f4*>(a.y + base + pstart);

        f4 v[VEC];
        float cnt, mean_t, m2_t;
        if (plen == PART) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) v[j] = ld_stream(xs + j * BLOCK + tid);
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                v[j] -= K;
                s0 += v[j].x;
                s1 += v[j].y;
                s2 += v[j].z;
                s3 += v[j].w;
            }
            cnt = (float)(4 * VEC);
            mean_t = ((s0 + s1) + (s2 + s3)) * (1.0f / (float)(4 * VEC));
            float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const f4 e = v[j] - mean_t;
                q0 = fmaf(e.x, e.x, q0);
                q1 = fmaf(e.y, e.y, q1);
                q2 = fmaf(e.z, e.z, q2);
                q3 = fmaf(e.w, e.w, q3);
            }
            m2_t = (q0 + q1) + (q2 + q3);
        } else {
            int nv = 0;
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int i = j * BLOCK + tid;
                if (i < nvec) {
                    v[j] = ld_stream(xs + i) - K;
                    s0 += v[j].x;
                    s1 += v[j].y;
                    s2 += v[j].z;
                    s3 += v[j].w;
                    ++nv;
                } else {
                    v[j] = f4{0.f, 0.f, 0.f, 0.f};
                }
            }
            cnt = (float)(4 * nv);
            mean_t = nv > 0 ? ((s0 + s1) + (s2 + s3)) / cnt : 0.f;
            float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                if (j * BLOCK + tid < nvec) {
                    const f4 e = v[j] - mean_t;
                    q0 = fmaf(e.x, e.x, q0);
                    q1 = fmaf(e.y, e.y, q1);
                    q2 = fmaf(e.z, e.z, q2);
                    q3 = fmaf(e.w, e.w, q3);
                }
            }
            m2_t = (q0 + q1) + (q2 + q3);
        }

        Stat st = wave_merge<kWave>(Stat{cnt, mean_t, m2_t});
        if (lane == 0) wstat[wid] = st;
        __syncthreads();

        if (wid == 0) {
            Stat w = lane < NW ? wstat[lane] : stat_empty();
            w = wave_merge<NW>(w);  // lanes 0..NW-1: this part's statistics

            if (P > 1) {
                unsigned long long* sl = a.slots + (size_t)slice * P * 2;
                if (lane == 0) {
                    xchg_store(sl + part * 2 + 0, kTag, w.mean);
                    xchg_store(sl + part * 2 + 1, kTag, w.m2);
                }
                Stat ps = stat_empty();
                if (lane < P) {
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
                    ps.n = prem <= 0 ? 0.f : (float)(prem < PART ? prem : PART);
                    ps.mean = __uint_as_float((uint32_t)w0);
                    ps.m2 = __uint_as_float((uint32_t)w1);
                }
                w = wave_merge<kMaxParts>(ps);  // parts merged in order 0..P-1
            }

            if (lane == 0) {
                const float var = w.m2 / w.n;
                const float rstd = rsqrtf(var + a.eps);
                const int64_t c = slice % a.C;
                const float g = a.gamma ? a.gamma[c] : 1.f;
                const float b = a.beta ? a.beta[c] : 0.f;
                fin[0] = w.mean;
                fin[1] = rstd * g;
                fin[2] = b;
                if (part == 0 && a.save_mean) a.save_mean[slice] = K + w.mean;
                if (part == 0 && a.save_invstd) a.save_invstd[slice] = rstd;
            }
        }
        __syncthreads();

        const float md = fin[0], sc = fin[1], sh = fin[2];
        if (plen == PART) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const f4 o = (v[j] - md) * sc + sh;
                st_stream(ys + j * BLOCK + tid, o);
            }
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int i = j * BLOCK + tid;
                if (i < nvec) st_stream(ys + i, (v[j] - md) * sc + sh);
            }
        }
    }
}

struct CfgEntry {
    ResidentCfg cfg;
    const void* fn;
};

#define NR_RES(B, V, W) \
    CfgEntry { ResidentCfg{B, V, B * 4 * V}, reinterpret_cast<const void*>(&inorm_resident_kernel<B, V, W>) }

// Ascending part length. waves_per_eu keeps the register budget at <= 128 VGPRs where two
// workgroups of the larger configurations should share a CU.
const CfgEntry kCfgs[] = {
    NR_RES(256, 1, 4),  NR_RES(256, 2, 4),  NR_RES(256, 4, 4), NR_RES(256, 8, 4),
    NR_RES(256, 16, 4), NR_RES(512, 16, 4), NR_RES(1024, 16, 4),
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

const void* cfg_fn(const ResidentCfg& c)
{
    for (int i = 0; i < kNumCfgs; ++i)
        if (kCfgs[i].cfg.block == c.block && kCfgs[i].cfg.vec == c.vec) return kCfgs[i].fn;
    return nullptr;
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
    return cus * per_cu;
}

hipError_t launch_resident(const ResidentCfg& cfg, const ResidentArgs& a, hipStream_t stream)
{
    const void* fn = cfg_fn(cfg);
    if (!fn) return hipErrorInvalidDeviceFunction;
    const int64_t units = a.slices * a.P;
    ResidentArgs args = a;
    void* params[] = {&args};
    if (a.P == 1) {
        const int64_t grid = units < 0x7fffffff ? units : 0x7fffffff;
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(cfg.block), params, 0, stream);
    }
    int64_t grid = resident_max_grid(cfg);
    if (grid > units) grid = units;
    grid -= grid % a.P;  // every round holds whole slices
    if (grid < a.P) return hipErrorCooperativeLaunchTooLarge;
    const hipError_t e = launch_fill_zero(a.slots, resident_slot_bytes(a.slices, a.P), stream);
    if (e != hipSuccess) return e;
    return hipLaunchCooperativeKernel(fn, dim3((unsigned)grid), dim3(cfg.block), params, 0, stream);
}

}  // namespace nr
