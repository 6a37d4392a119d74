// flat_norm.hip -- read-once instance normalization (and, further down, training-mode batch
// normalization) for slices whose length is not a multiple of 4, in a 16-byte aligned tensor: apart from the first, such slices start off 16-byte
// boundaries, so the read-once kernels of resident_norm.hip (16-byte accesses from each slice's
// start) do not apply. Short aligned slices (fewer than 1024 values) take it too: it sizes the
// lanes to the slice, where the smallest resident workgroup (256 threads) would mostly idle.
//
// IN2d page, statement of the op (and the IN3d page's InstanceNorm3d reading): per (n, c) slice
// of S values, mean and biased variance over the slice, y = (x - mean) / sqrt(var + eps), then
// y * gamma[c] + beta[c] when the affine parameters are given.
//
// One workgroup per slice. Of the aligned 16-byte blocks of the whole tensor that the slice
// [s*S, s*S + S) touches, those wholly inside it are spread over the threads (thread t holds
// whole blocks t, t + BLOCK, ... in registers) and read and written with 16-byte accesses; the
// slice's values in the partly covered first and last block (at most 3 each) are held by
// threads 0 and 1 and read and written with 4-byte accesses. No value outside the slice is
// written, and none is read except, for masked register slots, the tensor's first block: every
// value of x is read once and every value of y written once, and in place (y == x) no
// workgroup reads a value that another one writes. Slices of up to 1018 values share a
// 256-thread workgroup: each takes an aligned group of 4 to 64 lanes (several groups to a wave
// below 64 lanes), and "thread" above means lane of its group.
//
// Statistics as in the other kernels: values shifted by the slice's first value (the pivot),
// a two-pass (mean, M2) per thread over its registers, then pairwise (Chan) merges across the
// wave (fixed butterfly) and across the waves (wave 0, fixed order): deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace nr {
namespace {

// LANES == BLOCK: one slice per workgroup (cross-wave merge through LDS when BLOCK > 64).
// LANES < BLOCK (LANES <= 64): each aligned group of LANES lanes holds one slice (BLOCK / LANES
// slices per workgroup), merged by a butterfly inside the group; no LDS, no barrier.
template <int BLOCK, int VEC, int LANES>
__global__ __attribute__((amdgpu_flat_work_group_size(BLOCK, BLOCK))) void
flat_norm_kernel(const float* x, float* y, int64_t slices, int64_t C, int64_t S, float eps,
                 const float* gamma, const float* beta, float* save_mean, float* save_invstd)
{
    constexpr bool SUB = LANES < BLOCK;
    static_assert(SUB ? (BLOCK % kWave == 0 && LANES <= kWave && (LANES & (LANES - 1)) == 0)
                      : LANES == BLOCK,
                  "a slice takes a power-of-two group inside a wave, or the whole workgroup");
    constexpr int NW = BLOCK / kWave;
    __shared__ Stat wstat[SUB ? 1 : NW];
    __shared__ float coef[2];
    const int tid = threadIdx.x;
    const int gl = SUB ? tid % LANES : tid;  // lane within the slice's group
    const int64_t s = SUB ? (int64_t)blockIdx.x * (BLOCK / LANES) + tid / LANES : blockIdx.x;
    const bool live = !SUB || s < slices;    // groups past the last slice only join shuffles
    const int64_t start = live ? s * S : 0;
    const int len = (int)S;
    const int off0 = (int)(start & 3);       // the slice's first value inside its first block
    const int kw0 = off0 > 0 ? 1 : 0;        // first whole block (counted from the first block)
    const int kw1 = (off0 + len) >> 2;       // one past the last whole block
    const int nwb = live && kw1 > kw0 ? kw1 - kw0 : 0;
    // head: the slice's values in a partly covered first block; tail: those in a partly
    // covered last block that is not also the first
    const int nh = live && off0 > 0 ? min(4, off0 + len) - off0 : 0;
    const int nt = live && kw1 >= kw0 ? off0 + len - 4 * kw1 : 0;
    const float K = x[start];

    // Every load is issued unconditionally: an index past the whole blocks reads whole block 0
    // of the slice instead (block 0 of the tensor for a slice without whole blocks or a group
    // past the last slice; the tensor holds at least 4 values), and the value is masked below.
    const int64_t wb0 = ((start - off0) >> 2) + kw0;  // tensor block index of whole block 0
    const f4* xv = reinterpret_cast<const f4*>(x);
    f4 v[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int i = j * LANES + gl;
        v[j] = ld_stream(xv + (i < nwb ? wb0 + i : (nwb > 0 ? wb0 : 0)));
    }
    int ne = 0;
    int64_t eo = start;  // first edge value of this lane
    if (gl == 0) {
        ne = nh;
    } else if (gl == 1) {
        ne = nt;
        eo = start + len - nt;
    }
    float ev[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) ev[q] = ld_stream1(x + (q < ne ? eo + q : start));

    // Pivot-shifted values; registers past the last whole block become 0 and stay out of the
    // count.
    int cw = 0;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const bool in = j * LANES + gl < nwb;
        v[j] = in ? v[j] - K : f4{0.f, 0.f, 0.f, 0.f};
        cw += in;
        acc += v[j];
    }
    float sum = (acc.x + acc.y) + (acc.z + acc.w);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        ev[q] = q < ne ? ev[q] - K : 0.f;
        sum += ev[q];
    }
    const int cnt = 4 * cw + ne;
    const float fn = (float)cnt;
    const float m = cnt > 0 ? sum / fn : 0.f;
    f4 qa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const f4 d = v[j] - m;
        qa = j * LANES + gl < nwb ? qa + d * d : qa;
    }
    float q2 = (qa.x + qa.y) + (qa.z + qa.w);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const float d = ev[q] - m;
        q2 = q < ne ? fmaf(d, d, q2) : q2;
    }
    float sc, sh;
    if (SUB) {
        // every lane of the group ends with the slice's statistics
        const Stat w = wave_merge<LANES>(Stat{fn, m, q2});
        const float rstd = rsqrtf(w.m2 / w.n + eps);
        const int64_t c = live ? s % C : 0;
        const float gm = gamma ? gamma[c] : 1.f;
        const float bt = beta ? beta[c] : 0.f;
        sc = rstd * gm;
        sh = fmaf(-w.mean, sc, bt);
        if (live && gl == 0) {
            if (save_mean) save_mean[s] = K + w.mean;
            if (save_invstd) save_invstd[s] = rstd;
        }
    } else {
        const Stat st = wave_merge<kWave>(Stat{fn, m, q2});
        if (lane_id() == 0) wstat[tid / kWave] = st;
        __syncthreads();
        if (tid < kWave) {
            Stat w = lane_id() < NW ? wstat[lane_id()] : stat_empty();
            w = wave_merge<NW>(w);
            if (tid == 0) {
                const float rstd = rsqrtf(w.m2 / w.n + eps);
                const int64_t c = s % C;
                const float gm = gamma ? gamma[c] : 1.f;
                const float bt = beta ? beta[c] : 0.f;
                const float scl = rstd * gm;
                coef[0] = scl;
                coef[1] = fmaf(-w.mean, scl, bt);
                if (save_mean) save_mean[s] = K + w.mean;
                if (save_invstd) save_invstd[s] = rstd;
            }
        }
        __syncthreads();
        sc = coef[0];
        sh = coef[1];
    }
    f4* yv = reinterpret_cast<f4*>(y);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int i = j * LANES + gl;
        if (i < nwb) st_stream(yv + wb0 + i, v[j] * sc + sh);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
        if (q < ne) st_stream1(y + eo + q, fmaf(ev[q], sc, sh));
}

// Training-mode batch norm over slices with S % 4 != 0 in a 16-byte aligned tensor, for
// channels of up to ROUNDS * (256 / LANES) slices: one 256-thread workgroup per channel, which
// reads the channel once and writes it once. In round r, lane group g (LANES lanes) holds slice
// n = r * (256 / LANES) + g of the channel, as whole blocks and edge values like the kernel
// above. BN page, opening analysis: the batch statistics of a channel over all N slices (biased
// variance in the normalization, the unbiased one blended into the running variance), then
// y = ((x - mean) / sqrt(var + eps) * gamma[c] + beta[c]) * out_scale. The pivot is the
// channel's first value, as in the other batch-norm kernels.
template <int LANES, int VEC, int ROUNDS>
__global__ __launch_bounds__(256) void
flat_bn_kernel(const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps,
               const float* gamma, const float* beta, float out_scale, float* save_mean,
               float* save_invstd, float* running_mean, float* running_var, float momentum)
{
    constexpr int BLOCK = 256, G = BLOCK / LANES, NW = BLOCK / kWave;
    static_assert(LANES <= kWave && (LANES & (LANES - 1)) == 0, "lane groups inside a wave");
    __shared__ Stat wstat[NW];
    __shared__ float coef[2];
    const int tid = threadIdx.x, gl = tid % LANES, gi = tid / LANES;
    const int64_t c = blockIdx.x;
    const int len = (int)S;
    const float K = x[c * S];
    // Geometry of this lane's slice in round r; a group past the last slice gets no values
    // (its loads read the tensor's first block and the channel's first value, masked).
    struct Seg {
        int64_t wb0, eo;
        int nwb, ne;
    };
    auto seg = [&](int r) {
        const int64_t n = (int64_t)r * G + gi;
        const bool live = n < N;
        const int64_t start = live ? (n * C + c) * S : c * S;
        const int off0 = (int)(start & 3);
        const int kw0 = off0 > 0 ? 1 : 0, kw1 = (off0 + len) >> 2;
        Seg q;
        q.nwb = live && kw1 > kw0 ? kw1 - kw0 : 0;
        const int nh = live && off0 > 0 ? min(4, off0 + len) - off0 : 0;
        const int nt = live && kw1 >= kw0 ? off0 + len - 4 * kw1 : 0;
        q.wb0 = ((start - off0) >> 2) + kw0;
        q.ne = gl == 0 ? nh : (gl == 1 ? nt : 0);
        q.eo = gl == 1 ? start + len - nt : start;
        return q;
    };
    const f4* xv = reinterpret_cast<const f4*>(x);
    f4 v[ROUNDS][VEC];
    float ev[ROUNDS][3];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const Seg q = seg(r);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int i = j * LANES + gl;
            v[r][j] = ld_stream(xv + (i < q.nwb ? q.wb0 + i : (q.nwb > 0 ? q.wb0 : 0)));
        }
#pragma unroll
        for (int e = 0; e < 3; ++e) ev[r][e] = ld_stream1(x + (e < q.ne ? q.eo + e : c * S));
    }
    int cnt = 0;
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const Seg q = seg(r);
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const bool in = j * LANES + gl < q.nwb;
            v[r][j] = in ? v[r][j] - K : f4{0.f, 0.f, 0.f, 0.f};
            cnt += in ? 4 : 0;
            acc += v[r][j];
        }
        sum += (acc.x + acc.y) + (acc.z + acc.w);
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            ev[r][e] = e < q.ne ? ev[r][e] - K : 0.f;
            sum += ev[r][e];
        }
        cnt += q.ne;
    }
    const float fn = (float)cnt;
    const float m = cnt > 0 ? sum / fn : 0.f;
    float q2 = 0.f;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const Seg q = seg(r);
        f4 qa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const f4 d = v[r][j] - m;
            qa = j * LANES + gl < q.nwb ? qa + d * d : qa;
        }
        q2 += (qa.x + qa.y) + (qa.z + qa.w);
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            const float d = ev[r][e] - m;
            q2 = e < q.ne ? fmaf(d, d, q2) : q2;
        }
    }
    const Stat st = wave_merge<kWave>(Stat{fn, m, q2});
    if (lane_id() == 0) wstat[tid / kWave] = st;
    __syncthreads();
    if (tid < kWave) {
        Stat w = lane_id() < NW ? wstat[lane_id()] : stat_empty();
        w = wave_merge<NW>(w);
        if (tid == 0) {
            const float rstd = rsqrtf(w.m2 / w.n + eps);
            const float gm = gamma ? gamma[c] : 1.f;
            const float bt = beta ? beta[c] : 0.f;
            const float sc = rstd * gm * out_scale;
            coef[0] = sc;
            coef[1] = fmaf(-w.mean, sc, bt * out_scale);
            if (save_mean) save_mean[c] = K + w.mean;
            if (save_invstd) save_invstd[c] = rstd;
            if (running_mean) {
                running_mean[c] = (1.f - momentum) * running_mean[c] + momentum * (K + w.mean);
                running_var[c] = (1.f - momentum) * running_var[c] + momentum * (w.m2 / (w.n - 1.f));
            }
        }
    }
    __syncthreads();
    const float sc = coef[0], sh = coef[1];
    f4* yv = reinterpret_cast<f4*>(y);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const Seg q = seg(r);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int i = j * LANES + gl;
            if (i < q.nwb) st_stream(yv + q.wb0 + i, v[r][j] * sc + sh);
        }
#pragma unroll
        for (int e = 0; e < 3; ++e)
            if (e < q.ne) st_stream1(y + q.eo + e, fmaf(ev[r][e], sc, sh));
    }
}

struct FlatBnCfg {
    int lanes, vec, rounds;
};
// lanes x vec whole blocks per slice, (256 / lanes) x rounds slices per channel; at most 16
// registers a lane.
constexpr FlatBnCfg kFlatBnCfgs[] = {{4, 1, 8},  {4, 2, 8},  {16, 1, 8}, {8, 4, 4},
                                     {16, 4, 4}, {32, 4, 4}, {64, 4, 4}};

const FlatBnCfg* flat_bn_cfg(int64_t N, int64_t S)
{
    const int64_t need = (S + 6) / 4;
    for (const FlatBnCfg& c : kFlatBnCfgs)
        if ((int64_t)c.lanes * c.vec >= need && (int64_t)(256 / c.lanes) * c.rounds >= N) return &c;
    return nullptr;
}

struct FlatCfg {
    int block, vec, lanes;
};
// Ascending capacity (lanes x vec whole blocks per slice); a slice of S values spans at most
// (S + 6) / 4 blocks.
// Lane groups hold 4 blocks a lane once a slice needs more than 16: narrower groups with more
// loads in flight per lane keep more bytes in flight per wave (x[128,1024,14,14]: 0.046 ms
// against 0.071 with 64 lanes x 1 block). Up to 16 blocks, 16 lanes x 1 block measured faster
// than 4 x 4 (7 x 7 slices: 0.0135 against 0.0162 ms).
constexpr FlatCfg kFlatCfgs[] = {{256, 1, 4},  {256, 2, 4},   {256, 1, 16},  {256, 4, 8},
                                 {256, 4, 16}, {256, 4, 32},  {256, 4, 64},  {256, 4, 256},
                                 {256, 16, 256}, {512, 16, 512}, {1024, 16, 1024}};

}  // namespace

// The one-workgroup-per-channel form pays each workgroup's load, merge and store latency in
// sequence, so it is used only when the whole grid is resident at once: with 2048 channels of
// x[128,2048,7,7] (two batches of workgroups) it took 0.077 ms against 0.049 for the split path,
// with 512 channels 0.020 against 0.022.
bool flat_bn_fits(int64_t N, int64_t C, int64_t S)
{
    const FlatBnCfg* c = S % 4 != 0 ? flat_bn_cfg(N, S) : nullptr;
    if (!c) return false;
    const void* fn = nullptr;
#define NR_FLATBN_FN(L, V, R) \
    if (c->lanes == L && c->vec == V && c->rounds == R) fn = reinterpret_cast<const void*>(&flat_bn_kernel<L, V, R>);
    NR_FLATBN_FN(4, 1, 8)
    NR_FLATBN_FN(4, 2, 8)
    NR_FLATBN_FN(16, 1, 8)
    NR_FLATBN_FN(8, 4, 4)
    NR_FLATBN_FN(16, 4, 4)
    NR_FLATBN_FN(32, 4, 4)
    NR_FLATBN_FN(64, 4, 4)
#undef NR_FLATBN_FN
    int dev = 0, cus = 0, per_cu = 0;
    if (!fn || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess)
        return false;
    return C <= (int64_t)cus * per_cu;
}

hipError_t launch_flat_bn(const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps,
                          const float* gamma, const float* beta, float out_scale,
                          float* save_mean, float* save_invstd, float* running_mean,
                          float* running_var, float momentum, hipStream_t stream)
{
    const FlatBnCfg* c = flat_bn_cfg(N, S);
    if (!c || N < 1 || C < 1 || C > 0x7fffffffLL || N * C * S < 4) return hipErrorInvalidValue;
    const dim3 grid((unsigned)C), blk(256);
#define NR_FLATBN(L, V, R)                                                                        \
    if (c->lanes == L && c->vec == V && c->rounds == R) {                                         \
        flat_bn_kernel<L, V, R><<<grid, blk, 0, stream>>>(x, y, N, C, S, eps, gamma, beta,       \
                                                          out_scale, save_mean, save_invstd,     \
                                                          running_mean, running_var, momentum);  \
        return hipGetLastError();                                                                 \
    }
    NR_FLATBN(4, 1, 8)
    NR_FLATBN(4, 2, 8)
    NR_FLATBN(16, 1, 8)
    NR_FLATBN(8, 4, 4)
    NR_FLATBN(16, 4, 4)
    NR_FLATBN(32, 4, 4)
    NR_FLATBN(64, 4, 4)
#undef NR_FLATBN
    return hipErrorInvalidValue;
}

int64_t flat_norm_max_len() { return 4 * 1024 * 16 - 6; }

hipError_t launch_flat_norm(const float* x, float* y, int64_t slices, int64_t C, int64_t S,
                            float eps, const float* gamma, const float* beta, float* save_mean,
                            float* save_invstd, hipStream_t stream)
{
    if (S < 1 || S > flat_norm_max_len() || slices < 1 || slices > 0x7fffffffLL || slices * S < 4)
        return hipErrorInvalidValue;
    const int64_t need = (S + 6) / 4;
    for (const FlatCfg& c : kFlatCfgs) {
        if ((int64_t)c.lanes * c.vec < need) continue;
        const int64_t per = c.block / c.lanes;  // slices per workgroup
        const dim3 grid((unsigned)((slices + per - 1) / per)), blk(c.block);
#define NR_FLAT(B, V, L)                                                                          \
    if (c.block == B && c.vec == V && c.lanes == L) {                                             \
        flat_norm_kernel<B, V, L><<<grid, blk, 0, stream>>>(x, y, slices, C, S, eps, gamma, beta, \
                                                            save_mean, save_invstd);              \
        return hipGetLastError();                                                                 \
    }
        NR_FLAT(256, 1, 4)
        NR_FLAT(256, 2, 4)
        NR_FLAT(256, 1, 16)
        NR_FLAT(256, 4, 8)
        NR_FLAT(256, 4, 16)
        NR_FLAT(256, 4, 32)
        NR_FLAT(256, 4, 64)
        NR_FLAT(256, 4, 256)
        NR_FLAT(256, 16, 256)
        NR_FLAT(512, 16, 512)
        NR_FLAT(1024, 16, 1024)
#undef NR_FLAT
    }
    return hipErrorInvalidValue;
}

}  // namespace nr
