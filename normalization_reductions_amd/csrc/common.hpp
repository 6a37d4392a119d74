// common.hpp -- device building blocks shared by the gfx950 kernels of libnormred.
//
// Statistics are carried as (count, mean, M2) with M2 = sum of squared deviations from the
// mean. Partial statistics are combined with the pairwise (Chan et al.) update that the IN2d
// page (task l1_p34, its Welford kernel design) and the IN3d page (task l2_p79, its shared-
// memory tree of Welford states) both use:
//     n = na + nb,  d = mean_b - mean_a,  mean = mean_a + d*nb/n,  M2 = M2a + M2b + d^2*na*nb/n
// with an empty state (n = 0) acting as the identity.
//
// Wave reductions are written for 64-lane wavefronts: a butterfly over lane distances
// 1, 2, 4, ..., 32 in which both partners always merge (lower lane, upper lane) in that order,
// so every lane of a group ends with bit-identical results and the combine order is a fixed
// balanced tree over consecutive lanes -- deterministic from run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nr {

constexpr int kWave = 64;

typedef float f4 __attribute__((ext_vector_type(4)));

struct Stat {
    float n;     // element count (exact in fp32 up to 2^24)
    float mean;  // mean of the values (relative to the caller's pivot)
    float m2;    // sum of squared deviations from `mean`
};

__device__ __forceinline__ Stat stat_empty() { return Stat{0.f, 0.f, 0.f}; }

// Pairwise merge; `a` is always the lower-indexed range, `b` the higher one.
__device__ __forceinline__ Stat chan_merge(Stat a, Stat b)
{
    const float n = a.n + b.n;
    const float f = n > 0.f ? b.n / n : 0.f;  // weight of b
    const float d = b.mean - a.mean;
    Stat r;
    r.n = n;
    r.mean = fmaf(d, f, a.mean);
    r.m2 = a.m2 + b.m2 + d * d * a.n * f;
    return r;
}

// Rounded product that the compiler may not fuse into a following add. A chain's statistics
// and its normalize step both form u = c * pre_mul; on a constant channel (variance 0, so the
// deviation is multiplied by 1/sqrt(eps)) the two must round u the same way, and a fused
// fma(c, pm, -mean) keeps the product's rounding error that the statistics' mean dropped.
__device__ __forceinline__ float mul_rn(float a, float b)
{
#pragma clang fp contract(off)
    return a * b;
}
__device__ __forceinline__ f4 mul_rn(f4 a, float b)
{
#pragma clang fp contract(off)
    return a * b;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Butterfly over lane distances 1 .. WIDTH/2 (WIDTH a power of two <= 64). After it, every
// lane of each aligned group of WIDTH lanes holds the merge of the group, combined as a
// balanced tree over consecutive lanes.
template <int WIDTH>
__device__ __forceinline__ Stat wave_merge(Stat s)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < WIDTH; off <<= 1) {
        Stat o;
        o.n = __shfl_xor(s.n, off);
        o.mean = __shfl_xor(s.mean, off);
        o.m2 = __shfl_xor(s.m2, off);
        const bool upper = (lane & off) != 0;
        s = upper ? chan_merge(o, s) : chan_merge(s, o);
    }
    return s;
}

// Lane-strided merge of `total` items: lane l merges items l, l + WIDTH, l + 2 WIDTH, ... in
// that order. The loads of 8 items are issued together (indexes clamped, so the loads are
// unconditional) before their merges: one cache round trip per 8 items instead of one per item.
// load(q) returns the Stat of item q < total.
template <int WIDTH, class Load>
__device__ __forceinline__ Stat lane_strided_merge(int64_t total, Load load)
{
    constexpr int kB = 8;
    const int64_t lane = threadIdx.x & (WIDTH - 1);
    Stat st = stat_empty();
    for (int64_t q0 = lane; q0 < total; q0 += (int64_t)kB * WIDTH) {
        Stat v[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int64_t q = q0 + (int64_t)b * WIDTH;
            v[b] = load(q < total ? q : total - 1);
        }
#pragma unroll
        for (int b = 0; b < kB; ++b)
            if (q0 + (int64_t)b * WIDTH < total) st = chan_merge(st, v[b]);
    }
    return st;
}

// The same with a runtime stride R (a power of two) among R adjacent lanes: lane l merges
// items l % R, l % R + R, ... in that order.
template <class Load>
__device__ __forceinline__ Stat lane_strided_merge_by(int64_t total, int R, Load load)
{
    constexpr int kB = 8;
    const int64_t r = threadIdx.x & (R - 1);
    Stat st = stat_empty();
    for (int64_t q0 = r; q0 < total; q0 += (int64_t)kB * R) {
        Stat v[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int64_t q = q0 + (int64_t)b * R;
            v[b] = load(q < total ? q : total - 1);
        }
#pragma unroll
        for (int b = 0; b < kB; ++b)
            if (q0 + (int64_t)b * R < total) st = chan_merge(st, v[b]);
    }
    return st;
}

// Defaults of optional per-channel parameters (1 for the multipliers, 0 for a shift), read
// through the same unconditional global load as a given parameter: `*(p ? p + k : &kParamOne)`
// (never written; not const, which would place them in the constant address space and turn
// the loads into flat ones). A load under a branch is waited for at the branch's end, which
// would also wait for every load issued before it.
static __device__ float kParamOne = 1.f, kParamZero = 0.f;

// Plain-sum butterfly (all lanes end with the same fixed-order sum).
template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < WIDTH; off <<= 1) {
        const float o = __shfl_xor(v, off);
        v = (lane & off) ? (o + v) : (v + o);
    }
    return v;
}

// Streaming 16-byte accesses: each byte of x and y is touched once, so hint non-temporal.
__device__ __forceinline__ f4 ld_stream(const f4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(f4* p, f4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ float ld_stream1(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream1(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Exchange words between the workgroups of a group's parts: 64-bit, a tag in the high half and an fp32
// payload in the low half. They are only ever accessed with relaxed agent-scope atomics, so
// each word is read whole and coherently across the XCDs' L2s; a reader accepts a word only
// when its tag says it was written by the current launch.
__device__ __forceinline__ void xchg_store(unsigned long long* p, uint32_t tag, float v)
{
    const unsigned long long w =
        ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long xchg_load(unsigned long long* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Upper bound on polling rounds in an exchange wait. A round is a short sleep plus two
// device-coherent loads, so 2^22 rounds is far beyond any legitimate wait (the siblings a
// waiter needs are held by running workgroups whenever 16 or more of the grid run); it keeps a
// starved or broken launch from spinning forever: the wait gives up and raises a sticky flag.
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint32_t kFlagSpinTimeout = 1u;

__device__ __forceinline__ void raise_flag(uint32_t* flags, uint32_t bit)
{
    __hip_atomic_fetch_or(flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace nr
