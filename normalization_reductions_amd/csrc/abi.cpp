// abi.cpp -- the extern "C" boundary of libnormred: argument validation, variant planning,
// workspace layout and kernel dispatch. Validation never touches the HIP runtime, so every
// rejection path works (and is tested) on machines without a GPU.
#include "normred.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "internal.hpp"

using namespace nr;

namespace {

thread_local std::string t_err;

nr_status vfail(nr_status s, const char* fmt, va_list ap)
{
    char buf[512];
    vsnprintf(buf, sizeof(buf), fmt, ap);
    t_err = buf;
    return s;
}

nr_status fail(nr_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nr_status fail(nr_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vfail(s, fmt, ap);
    va_end(ap);
    return s;
}

}  // namespace

nr_status nr::set_error(nr_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vfail(s, fmt, ap);
    va_end(ap);
    return s;
}

namespace {

nr_status hip_fail(hipError_t e, const char* where)
{
    return fail(NR_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Total element count N*C*S (and its byte size) without overflow. N and C may be 0 when
// allow_empty (an empty batch is a no-op); S must be >= 1 (a statistic over nothing is undefined).
nr_status check_sizes(int64_t N, int64_t C, int64_t S, int64_t* total, const char* fn,
                      bool allow_empty = true)
{
    const int64_t lo = allow_empty ? 0 : 1;
    if (N < lo || C < lo || S < 1)
        return fail(NR_ERR_INVALID_ARG, "%s: sizes out of range (N=%lld C=%lld S=%lld)", fn,
                    (long long)N, (long long)C, (long long)S);
    int64_t nc = 0, t = 0, bytes = 0;
    if (!mul_ok(N, C, &nc) || !mul_ok(nc, S, &t) || !mul_ok(t, 4, &bytes))
        return fail(NR_ERR_INVALID_ARG, "%s: N*C*S overflows", fn);
    *total = t;
    return NR_OK;
}

nr_status check_eps(float eps, const char* fn)
{
    if (!std::isfinite(eps) || eps < 0.f) return fail(NR_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
    return NR_OK;
}

// Optional per-channel fp32 vector: NULL or 4-byte aligned.
nr_status check_opt(const void* p, const char* name, const char* fn)
{
    if (p && !aligned(p, 4)) return fail(NR_ERR_MISALIGNED, "%s: %s is not 4-byte aligned", fn, name);
    return NR_OK;
}

bool ranges_partially_overlap(const float* a, const float* b, int64_t n)
{
    if (a == b) return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    const uintptr_t len = (uintptr_t)n * 4u;
    return pa < pb + len && pb < pa + len;
}

// ---------------------------------------------------------------------------------------------
// Instance-norm planning.
// ---------------------------------------------------------------------------------------------
// Optional override of the resident configuration, "block,vec" (tuning, tests and benchmarks
// only; read on every call).
bool resident_override(int* block, int* vec)
{
    const char* e = getenv("NORMRED_RESIDENT_CFG");
    int b = 0, v = 0;
    if (e && sscanf(e, "%d,%d", &b, &v) == 2 && b > 0 && v > 0) {
        *block = b;
        *vec = v;
        return true;
    }
    return false;
}

// Pick a read-once configuration and part count for groups of L values of the given kind.
// Without an override: groups that fit a workgroup of up to 512 threads (<= 32K values) take
// the smallest single-workgroup configuration of the kind that holds them (measured faster
// than splitting such groups); larger groups take the pipelined kernel with 64 KiB parts (256
// threads x 16 float4), or 128 KiB parts past 32 of those. (For 64K-value slices, 4 pipelined
// parts measured 6 % faster than one 1024-thread workgroup per slice.)
// Grouped kinds (batch norm) need L < 2^21 for their index arithmetic.
bool choose_resident(int64_t L, bool grouped, bool chain, int* cfg_idx, int* P)
{
    if (grouped && L >= (1 << 21)) return false;
    const int n = resident_cfg_count();
    int ob, ov;
    const bool over = resident_override(&ob, &ov);
    for (int i = 0; i < n; ++i) {
        const ResidentCfg c = resident_cfg(i);
        if (c.grouped != grouped || c.chain != chain) continue;
        if (over && (c.block != ob || c.vec != ov)) continue;
        const int64_t p = (L + c.part_len - 1) / c.part_len;
        if (!c.pipelined) {
            if (p != 1 || (!over && c.block > 512)) continue;
        } else {
            if (p < 2 || p > kMaxParts) continue;
            if (!over && c.vec != 16) continue;
        }
        *cfg_idx = i;
        *P = (int)p;
        return true;
    }
    return false;
}

// Longest aligned slice (S % 4 == 0) that instance norm gives the flat one-workgroup kernel.
constexpr int64_t kFlatShortLen = 1020;

// Could a read-once configuration of this kind need the exchange regions for groups of L?
bool may_need_exchange(int64_t L, bool grouped)
{
    if (L <= 1024 || (grouped && L >= (1 << 21))) return false;
    int64_t biggest = 0;
    for (int i = 0; i < resident_cfg_count(); ++i)
        if (resident_cfg(i).pipelined && resident_cfg(i).part_len > biggest) biggest = resident_cfg(i).part_len;
    return L <= (int64_t)kMaxParts * biggest;
}

// Fill the fields of ResidentArgs that every kind shares.
ResidentArgs resident_args(const float* x, float* y, int64_t N, int64_t C, int64_t S, bool batch,
                           int P, float eps, const float* gamma, const float* beta,
                           float out_scale, float* save_mean, float* save_invstd, void* ws,
                           size_t exch_off, bool exch)
{
    ResidentArgs a{};
    a.x = x;
    a.y = y;
    a.S = S;
    a.C = C;
    a.groups = batch ? C : N * C;
    a.L = batch ? N * S : S;
    a.div_magic = resident_div_magic(S);
    a.batch = batch ? 1 : 0;
    a.P = P;
    a.eps = eps;
    a.gamma = gamma;
    a.beta = beta;
    a.out_scale = out_scale;
    a.save_mean = save_mean;
    a.save_invstd = save_invstd;
    a.counter = exch ? reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + exch_off) : nullptr;
    a.slots = exch ? reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + exch_off + kCounterBytes)
                   : nullptr;
    a.flags = reinterpret_cast<uint32_t*>(ws);
    return a;
}

struct InormLayout {
    size_t slots = 0, partials = 0, stats = 0, bytes = 0;
    bool exchange = false;
    SplitGeom sg;
};

InormLayout inorm_layout(int64_t N, int64_t C, int64_t S, bool vec)
{
    InormLayout L;
    const int64_t slices = N * C;
    size_t off = kHeaderBytes;
    L.exchange = S % 4 == 0 && may_need_exchange(S, false);
    if (L.exchange) {
        L.slots = off;  // counter, then slots
        off = align_up(off + resident_ws_bytes(slices, kMaxParts), kWsAlign);
    }
    L.sg = split_geometry(N, C, S, false, vec);
    L.partials = off;
    off = align_up(off + (size_t)(slices * L.sg.chunks) * sizeof(float2), kWsAlign);
    L.stats = off;
    off = align_up(off + (size_t)slices * sizeof(GroupStat), kWsAlign);
    L.bytes = off;
    return L;
}

template <typename T>
T* ws_at(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

nr_status check_workspace(void* ws, size_t have, size_t need, const char* fn)
{
    if (!ws) return fail(NR_ERR_WORKSPACE, "%s: workspace is NULL (need %zu bytes)", fn, need);
    if (!aligned(ws, kWsAlign)) return fail(NR_ERR_MISALIGNED, "%s: workspace must be 256-byte aligned", fn);
    if (have < need)
        return fail(NR_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, have, need);
    return NR_OK;
}

nr_status run_split(const SplitGeom& g, const float* x, float* y, float eps, const float* gamma,
                    const float* beta, float out_scale, float* save_mean, float* save_invstd,
                    RunningStats run, float2* partials, GroupStat* stats, hipStream_t stream,
                    const char* fn)
{
    if (g.slices * g.chunks > 0x7fffffffLL)
        return fail(NR_ERR_UNSUPPORTED, "%s: %lld slices x %lld chunks exceed one launch", fn,
                    (long long)g.slices, (long long)g.chunks);
    hipError_t e = launch_split_stats(g, x, nullptr, partials, eps, stats, save_mean, save_invstd,
                                      run, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    e = launch_split_apply(g, x, y, stats, gamma, beta, out_scale, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return NR_OK;
}

// Validate an optional running-statistics update: both buffers or neither, 4-byte aligned,
// momentum in [0, 1], at least two values per channel (the unbiased variance divides by n - 1).
nr_status check_running(const float* rm, const float* rv, float momentum, int64_t count,
                        const char* fn)
{
    if ((rm == nullptr) != (rv == nullptr))
        return fail(NR_ERR_INVALID_ARG, "%s: running_mean and running_var must both be given or both be NULL", fn);
    if (!rm) return NR_OK;
    if (!aligned(rm, 4) || !aligned(rv, 4))
        return fail(NR_ERR_MISALIGNED, "%s: running statistics must be 4-byte aligned", fn);
    if (!std::isfinite(momentum) || momentum < 0.f || momentum > 1.f)
        return fail(NR_ERR_INVALID_ARG, "%s: momentum must be in [0, 1]", fn);
    if (count < 2)
        return fail(NR_ERR_INVALID_ARG, "%s: running variance needs >= 2 values per channel", fn);
    return NR_OK;
}

size_t bn_layout(int64_t N, int64_t C, int64_t S, bool vec, SplitGeom* g, size_t* exch,
                 size_t* partials, size_t* stats)
{
    *g = split_geometry(N, C, S, true, vec);
    size_t off = kHeaderBytes;
    *exch = 0;
    if (S % 4 == 0 && may_need_exchange(N * S, true)) {
        *exch = off;
        off = align_up(off + resident_ws_bytes(C, kMaxParts), kWsAlign);
    }
    *partials = off;
    off = align_up(off + (size_t)(g->slices * g->chunks) * sizeof(float2), kWsAlign);
    *stats = off;
    off = align_up(off + (size_t)C * sizeof(GroupStat), kWsAlign);
    return off;
}

// ---------------------------------------------------------------------------------------------
// Conv chain planning.
// ---------------------------------------------------------------------------------------------
nr_status check_desc(const nr_conv_norm_desc* d, ConvGeom* g, const char* fn)
{
    if (!d) return fail(NR_ERR_INVALID_ARG, "%s: descriptor is NULL", fn);
    if (d->spatial_dims != 2 && d->spatial_dims != 3)
        return fail(NR_ERR_INVALID_ARG, "%s: spatial_dims must be 2 or 3", fn);
    if (d->ksize != 3) return fail(NR_ERR_UNSUPPORTED, "%s: only ksize 3 is implemented (got %d)", fn, d->ksize);
    if (d->N < 0 || d->C_in < 1 || d->C_out < 1)
        return fail(NR_ERR_INVALID_ARG, "%s: need N >= 0, C_in >= 1, C_out >= 1", fn);
    const int64_t D = d->spatial_dims == 3 ? d->in_d : 1;
    if (d->in_h < 3 || d->in_w < 3 || (d->spatial_dims == 3 && d->in_d < 3))
        return fail(NR_ERR_INVALID_ARG, "%s: input extent must be >= 3 along each spatial axis", fn);
    if (d->norm != NR_NORM_BATCH_TRAIN && d->norm != NR_NORM_INSTANCE)
        return fail(NR_ERR_INVALID_ARG, "%s: norm must be NR_NORM_BATCH_TRAIN or NR_NORM_INSTANCE", fn);
    nr_status s = check_eps(d->eps, fn);
    if (s != NR_OK) return s;
    if (!std::isfinite(d->out_scale)) return fail(NR_ERR_INVALID_ARG, "%s: out_scale must be finite", fn);
    if (d->clamp != 0 && d->clamp != 1) return fail(NR_ERR_INVALID_ARG, "%s: clamp must be 0 or 1", fn);
    if (d->clamp && !(d->clamp_lo <= d->clamp_hi))
        return fail(NR_ERR_INVALID_ARG, "%s: clamp_lo must be <= clamp_hi", fn);
    if (d->reduce_max_c != 0 && d->reduce_max_c != 1)
        return fail(NR_ERR_INVALID_ARG, "%s: reduce_max_c must be 0 or 1", fn);
    if ((s = check_opt(d->pre_mul, "pre_mul", fn)) != NR_OK) return s;
    if ((s = check_opt(d->gamma, "gamma", fn)) != NR_OK) return s;
    if ((s = check_opt(d->beta, "beta", fn)) != NR_OK) return s;
    if ((s = check_opt(d->post_mul, "post_mul", fn)) != NR_OK) return s;
    if (d->running_mean || d->running_var) {
        if (d->norm != NR_NORM_BATCH_TRAIN)
            return fail(NR_ERR_INVALID_ARG, "%s: running statistics need NR_NORM_BATCH_TRAIN", fn);
        const int64_t per_channel = d->N * (d->spatial_dims == 3 ? d->in_d - 2 : 1) *
                                    (d->in_h - 2) * (d->in_w - 2);
        if ((s = check_running(d->running_mean, d->running_var, d->momentum,
                               d->N == 0 ? 2 : per_channel, fn)) != NR_OK)
            return s;
    }
    ConvGeom c;
    c.dims = d->spatial_dims;
    c.N = d->N;
    c.Cin = d->C_in;
    c.Cout = d->C_out;
    c.D = D;
    c.H = d->in_h;
    c.W = d->in_w;
    c.OD = d->spatial_dims == 3 ? D - 2 : 1;
    c.OH = d->in_h - 2;
    c.OW = d->in_w - 2;
    int64_t t = 0, sp = 0, nc = 0;
    if (!mul_ok(c.OD, c.OH, &t) || !mul_ok(t, c.OW, &sp) || !mul_ok(c.N, c.Cout, &nc) ||
        !mul_ok(nc, sp, &t) || !mul_ok(t, 4, &t))
        return fail(NR_ERR_INVALID_ARG, "%s: output size overflows", fn);
    int64_t in_t = 0;
    if (!mul_ok(c.N, c.Cin, &in_t) || !mul_ok(in_t, D, &in_t) || !mul_ok(in_t, c.H, &in_t) ||
        !mul_ok(in_t, c.W, &in_t) || !mul_ok(in_t, 4, &in_t))
        return fail(NR_ERR_INVALID_ARG, "%s: input size overflows", fn);
    c.SP = sp;
    if (c.N > 65535 || (c.Cout + 15) / 16 > 65535 || (sp + 255) / 256 > 0x7fffffffLL)
        return fail(NR_ERR_UNSUPPORTED, "%s: shape exceeds the launch grid limits", fn);
    if (d->channels_last != 0 && d->channels_last != 1)
        return fail(NR_ERR_INVALID_ARG, "%s: channels_last must be 0 or 1", fn);
    c.cl = d->channels_last;
    if (c.cl && c.Cout > 256)
        return fail(NR_ERR_UNSUPPORTED, "%s: channels_last supports C_out <= 256", fn);
    *g = c;
    return NR_OK;
}

struct ChainLayout {
    bool resident = false;  // normalize in place in `out` with a read-once kernel
    bool recompute = false; // batch norm by recomputing the conv (2-D matrix producer shape)
    int cfg_idx = -1, P = 0;
    size_t exch = 0, c8part = 0, c8stats = 0;
    size_t cbuf = 0, partials = 0, stats = 0, bytes = 0;
    int64_t ring_J = 0;     // instance norm: slots of the ring producer's own statistics (0: none)
    SplitGeom sg;
    ClGeom cg;              // channels last
};

// Two plans. Without the max over channels and with S % 4 == 0 the conv writes its output
// straight into `out` and a read-once kernel normalizes it in place (workspace: exchange slots
// only). Otherwise the conv output goes to the workspace, statistics take the split path and
// the chain epilogue writes `out`.
ChainLayout chain_layout(const ConvGeom& g, bool batch, bool reduce_max_c)
{
    ChainLayout L;
    size_t off = kHeaderBytes;
    const int64_t groups = batch ? g.Cout : g.N * g.Cout;
    // instance norm on a ring producer shape: the producer takes the statistics of its output
    // itself ([N][J][C_out] partials), so no pass re-reads the conv output for them
    L.ring_J = batch ? 0 : ring_stats_slots(g);
    if (g.cl) {
        // channels last: conv output staged only for the max over channels (else written to
        // `out` and normalized in place), partials per (n, chunk, k) or the ring producer's
        // slots, group statistics
        L.cg = cl_geometry(g.N, g.Cout, g.SP, batch);
        if (L.ring_J > 0) {
            L.cg.chunk = 0;  // the slots stand in for the chunks
            L.cg.chunks = L.ring_J;
        }
        if (reduce_max_c) {
            L.cbuf = off;
            off = align_up(off + (size_t)(g.N * g.Cout * g.SP) * sizeof(float), kWsAlign);
        }
        L.partials = off;
        off = align_up(off + cl_partials_bytes(L.cg), kWsAlign);
        L.stats = off;
        off = align_up(off + (size_t)groups * sizeof(GroupStat), kWsAlign);
        L.bytes = off;
        return L;
    }
    const int64_t len = batch ? g.N * g.SP : g.SP;
    if (batch && !reduce_max_c && conv2d_c8_shape(g)) {
        // batch norm on the 2-D matrix producer's shape: statistics pass, merge, and the conv
        // again with the chain epilogue (no conv output in HBM). The read-once plan's exchange
        // slots follow, for calls whose pointers the producer cannot take.
        L.recompute = true;
        const int64_t G = conv2d_c8_grid_bound(g);
        L.c8part = off;
        off = align_up(off + (size_t)(g.Cout * G) * sizeof(float4), kWsAlign);
        L.c8stats = off;  // the published statistics: [C_out][2] tagged 64-bit words
        off = align_up(off + (size_t)g.Cout * 2 * sizeof(unsigned long long), kWsAlign);
    }
    if (!reduce_max_c && g.SP % 4 == 0 && choose_resident(len, batch, true, &L.cfg_idx, &L.P) &&
        groups * L.P <= 0xF0000000LL && groups <= 0x7fffffffLL) {
        L.resident = true;
        L.exch = off;
        off = align_up(off + resident_ws_bytes(groups, L.P), kWsAlign);
        L.bytes = off;
        return L;
    }
    L.cbuf = off;
    off = align_up(off + (size_t)(g.N * g.Cout * g.SP) * sizeof(float), kWsAlign);
    L.partials = off;
    if (L.ring_J > 0) {
        off = align_up(off + (size_t)(g.N * L.ring_J * g.Cout) * sizeof(float4), kWsAlign);
    } else {
        L.sg = split_geometry(g.N, g.Cout, g.SP, batch, g.SP % 4 == 0);
        off = align_up(off + (size_t)(L.sg.slices * L.sg.chunks) * sizeof(float2), kWsAlign);
    }
    L.stats = off;
    off = align_up(off + (size_t)groups * sizeof(GroupStat), kWsAlign);
    L.bytes = off;
    return L;
}

}  // namespace

// =============================================================================================
// Exported entry points.
// =============================================================================================
extern "C" {

__attribute__((visibility("default"))) const char* nr_last_error(void) { return t_err.c_str(); }

__attribute__((visibility("default"))) const char* nr_version(void) { return "normred 0.1.0 gfx950"; }

__attribute__((visibility("default"))) size_t inorm_workspace_size(int64_t N, int64_t C, int64_t S)
{
    int64_t total = 0;
    if (check_sizes(N, C, S, &total, "inorm_workspace_size") != NR_OK) return 0;
    // the vector and scalar split geometries are identical in size
    return inorm_layout(N, C, S, true).bytes;
}

__attribute__((visibility("default"))) nr_status inorm_forward_ex(
    const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps, const float* gamma,
    const float* beta, float* save_mean, float* save_invstd, void* workspace,
    size_t workspace_bytes, int variant, hipStream_t stream)
{
    static const char* fn = "inorm_forward";
    int64_t total = 0;
    nr_status s = check_sizes(N, C, S, &total, fn);
    if (s != NR_OK) return s;
    if (variant != NR_VARIANT_AUTO && variant != NR_VARIANT_RESIDENT && variant != NR_VARIANT_SPLIT)
        return fail(NR_ERR_INVALID_ARG, "%s: unknown variant %d", fn, variant);
    if (total == 0) return NR_OK;  // empty batch: nothing is read or written
    if (!x || !y) return fail(NR_ERR_INVALID_ARG, "%s: x and y must be non-NULL", fn);
    if (!aligned(x, 4) || !aligned(y, 4)) return fail(NR_ERR_MISALIGNED, "%s: x and y must be 4-byte aligned", fn);
    if (ranges_partially_overlap(x, y, total))
        return fail(NR_ERR_INVALID_ARG, "%s: x and y overlap without being the same buffer", fn);
    if ((gamma == nullptr) != (beta == nullptr))
        return fail(NR_ERR_INVALID_ARG, "%s: gamma and beta must both be given or both be NULL", fn);
    if ((s = check_eps(eps, fn)) != NR_OK) return s;
    if ((s = check_opt(gamma, "gamma", fn)) != NR_OK) return s;
    if ((s = check_opt(beta, "beta", fn)) != NR_OK) return s;
    if ((s = check_opt(save_mean, "save_mean", fn)) != NR_OK) return s;
    if ((s = check_opt(save_invstd, "save_invstd", fn)) != NR_OK) return s;

    const bool vec = aligned(x, 16) && aligned(y, 16) && S % 4 == 0;
    const InormLayout L = inorm_layout(N, C, S, vec);
    if ((s = check_workspace(workspace, workspace_bytes, L.bytes, fn)) != NR_OK) return s;

    int cfg_idx = -1, P = 0;
    const bool res_ok = vec && choose_resident(S, false, false, &cfg_idx, &P) && (P == 1 || L.exchange);
    // One workgroup per slice sized to it (flat_norm.hip): the read-once form for slices off
    // 16-byte boundaries (faster than the split path from S = 7 up), and for short aligned
    // slices, which the smallest resident workgroup (256 threads) mostly leaves idle: 1.7-3.4x
    // faster up to S = 768, as fast or slower from S = 1024.
    const bool flat_ok = aligned(x, 16) && aligned(y, 16) && S <= flat_norm_max_len() &&
                         N * C <= 0x7fffffffLL && total >= 4;
    const bool flat_pref = flat_ok && (S % 4 != 0 || S <= kFlatShortLen);
    bool use_res = false, use_flat = false;
    if (variant == NR_VARIANT_RESIDENT) {
        if (!res_ok && !flat_ok)
            return fail(NR_ERR_UNSUPPORTED,
                        "%s: the resident variant needs 16-byte aligned x/y and either S %% 4 == 0 "
                        "with S <= %d, or S <= %lld (S=%lld)", fn, kMaxParts * 32768,
                        (long long)flat_norm_max_len(), (long long)S);
        use_flat = flat_pref || !res_ok;
        use_res = !use_flat;
    } else if (variant == NR_VARIANT_AUTO) {
        use_flat = flat_pref;
        use_res = !use_flat && res_ok;
    }

    if (use_flat) {
        const hipError_t e = launch_flat_norm(x, y, N * C, C, S, eps, gamma, beta, save_mean,
                                              save_invstd, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    if (use_res) {
        if (N * C * P > 0xF0000000LL || N * C > 0x7fffffffLL)  // counter headroom, grid limit
            return fail(NR_ERR_UNSUPPORTED, "%s: too many slices for the resident variant", fn);
        const ResidentArgs a = resident_args(x, y, N, C, S, false, P, eps, gamma, beta, 1.0f,
                                             save_mean, save_invstd, workspace, L.slots, L.exchange);
        const hipError_t e = launch_resident(resident_cfg(cfg_idx), a, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    return run_split(L.sg, x, y, eps, gamma, beta, 1.0f, save_mean, save_invstd, RunningStats{},
                     ws_at<float2>(workspace, L.partials), ws_at<GroupStat>(workspace, L.stats),
                     stream, fn);
}

__attribute__((visibility("default"))) nr_status inorm_forward(
    const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps, const float* gamma,
    const float* beta, float* save_mean, float* save_invstd, void* workspace,
    size_t workspace_bytes, hipStream_t stream)
{
    return inorm_forward_ex(x, y, N, C, S, eps, gamma, beta, save_mean, save_invstd, workspace,
                            workspace_bytes, NR_VARIANT_AUTO, stream);
}

__attribute__((visibility("default"))) size_t bn_train_workspace_size(int64_t N, int64_t C, int64_t S)
{
    int64_t total = 0;
    if (N < 1 || check_sizes(N, C, S, &total, "bn_train_workspace_size") != NR_OK) return 0;
    SplitGeom g;
    size_t ex, p, st;
    return bn_layout(N, C, S, true, &g, &ex, &p, &st);
}

__attribute__((visibility("default"))) nr_status bn_train_forward_ex(
    const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps, const float* gamma,
    const float* beta, float out_scale, float* save_mean, float* save_invstd, float momentum,
    float* running_mean, float* running_var, void* workspace, size_t workspace_bytes,
    hipStream_t stream)
{
    static const char* fn = "bn_train_forward";
    if (N < 1) return fail(NR_ERR_INVALID_ARG, "%s: batch statistics need N >= 1", fn);
    int64_t total = 0;
    nr_status s = check_sizes(N, C, S, &total, fn);
    if (s != NR_OK) return s;
    if (total == 0) return NR_OK;  // no channels: nothing is read or written
    if (!x || !y) return fail(NR_ERR_INVALID_ARG, "%s: x and y must be non-NULL", fn);
    if (!aligned(x, 4) || !aligned(y, 4)) return fail(NR_ERR_MISALIGNED, "%s: x and y must be 4-byte aligned", fn);
    if (ranges_partially_overlap(x, y, total))
        return fail(NR_ERR_INVALID_ARG, "%s: x and y overlap without being the same buffer", fn);
    if ((gamma == nullptr) != (beta == nullptr))
        return fail(NR_ERR_INVALID_ARG, "%s: gamma and beta must both be given or both be NULL", fn);
    if ((s = check_eps(eps, fn)) != NR_OK) return s;
    if (!std::isfinite(out_scale)) return fail(NR_ERR_INVALID_ARG, "%s: out_scale must be finite", fn);
    if ((s = check_opt(gamma, "gamma", fn)) != NR_OK) return s;
    if ((s = check_opt(beta, "beta", fn)) != NR_OK) return s;
    if ((s = check_opt(save_mean, "save_mean", fn)) != NR_OK) return s;
    if ((s = check_opt(save_invstd, "save_invstd", fn)) != NR_OK) return s;
    if ((s = check_running(running_mean, running_var, momentum, N * S, fn)) != NR_OK) return s;
    const RunningStats run{running_mean, running_var, momentum};
    const bool vec = aligned(x, 16) && aligned(y, 16) && S % 4 == 0;
    SplitGeom g;
    size_t off_x, off_p, off_s;
    const size_t need = bn_layout(N, C, S, vec, &g, &off_x, &off_p, &off_s);
    if ((s = check_workspace(workspace, workspace_bytes, need, fn)) != NR_OK) return s;
    // slices off 16-byte boundaries, channels that one workgroup holds: read once (flat_norm.hip)
    if (S % 4 != 0 && aligned(x, 16) && aligned(y, 16) && flat_bn_fits(N, C, S) &&
        C <= 0x7fffffffLL && total >= 4) {
        const hipError_t e = launch_flat_bn(x, y, N, C, S, eps, gamma, beta, out_scale, save_mean,
                                            save_invstd, running_mean, running_var, momentum,
                                            stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    int cfg_idx = -1, P = 0;
    if (vec && choose_resident(N * S, true, false, &cfg_idx, &P) && (P == 1 || off_x != 0) &&
        C * P <= 0xF0000000LL && C <= 0x7fffffffLL) {
        ResidentArgs a = resident_args(x, y, N, C, S, true, P, eps, gamma, beta, out_scale,
                                       save_mean, save_invstd, workspace, off_x, off_x != 0);
        a.running_mean = running_mean;
        a.running_var = running_var;
        a.momentum = momentum;
        const hipError_t e = launch_resident(resident_cfg(cfg_idx), a, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    return run_split(g, x, y, eps, gamma, beta, out_scale, save_mean, save_invstd, run,
                     ws_at<float2>(workspace, off_p), ws_at<GroupStat>(workspace, off_s), stream, fn);
}

__attribute__((visibility("default"))) nr_status bn_train_forward(
    const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps, const float* gamma,
    const float* beta, float out_scale, float* save_mean, float* save_invstd, void* workspace,
    size_t workspace_bytes, hipStream_t stream)
{
    return bn_train_forward_ex(x, y, N, C, S, eps, gamma, beta, out_scale, save_mean, save_invstd,
                               0.f, nullptr, nullptr, workspace, workspace_bytes, stream);
}

__attribute__((visibility("default"))) size_t conv_norm_epilogue_workspace_size(const nr_conv_norm_desc* d)
{
    ConvGeom g;
    if (check_desc(d, &g, "conv_norm_epilogue_workspace_size") != NR_OK) return 0;
    return chain_layout(g, d->norm == NR_NORM_BATCH_TRAIN, d->reduce_max_c != 0).bytes;
}

__attribute__((visibility("default"))) nr_status conv_norm_epilogue_forward(
    const nr_conv_norm_desc* d, const float* x, const float* w, const float* b, float* out,
    void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    static const char* fn = "conv_norm_epilogue_forward";
    ConvGeom g;
    nr_status s = check_desc(d, &g, fn);
    if (s != NR_OK) return s;
    if (g.N == 0) return NR_OK;  // empty batch: nothing is read or written
    if (!x || !w || !out) return fail(NR_ERR_INVALID_ARG, "%s: x, w and out must be non-NULL", fn);
    if (!aligned(x, 4) || !aligned(w, 4) || !aligned(out, 4) || (b && !aligned(b, 4)))
        return fail(NR_ERR_MISALIGNED, "%s: tensors must be 4-byte aligned", fn);
    const bool batch = d->norm == NR_NORM_BATCH_TRAIN;
    const ChainLayout L = chain_layout(g, batch, d->reduce_max_c != 0);
    if ((s = check_workspace(workspace, workspace_bytes, L.bytes, fn)) != NR_OK) return s;
    if (g.cl) {
        if (L.cg.N * L.cg.chunks > 0x7fffffffLL || L.cg.chunks > 0x7fffffffLL)
            return fail(NR_ERR_UNSUPPORTED, "%s: too many statistics chunks for one launch", fn);
        float* c = d->reduce_max_c ? ws_at<float>(workspace, L.cbuf) : out;
        float4* part = ws_at<float4>(workspace, L.partials);
        GroupStat* stats = ws_at<GroupStat>(workspace, L.stats);
        hipError_t e;
        if (L.ring_J > 0) {
            e = launch_conv_k3_stats(g, x, w, b, c, RingStats{part, d->pre_mul, L.ring_J}, stream);
        } else {
            e = launch_conv_k3(g, x, w, b, c, stream);
            if (e == hipSuccess)
                e = launch_cl_stats(L.cg, c, d->pre_mul, part, d->eps, stats,
                                    RunningStats{d->running_mean, d->running_var, d->momentum},
                                    stream);
        }
        if (e != hipSuccess) return hip_fail(e, fn);
        ChainArgs a;
        a.c = c;
        a.out = out;
        a.N = g.N;
        a.Cout = g.Cout;
        a.SP = g.SP;
        a.batch = batch;
        a.stats = stats;
        a.pre_mul = d->pre_mul;
        a.gamma = d->gamma;
        a.beta = d->beta;
        a.out_scale = d->out_scale;
        a.clamp = d->clamp;
        a.lo = d->clamp_lo;
        a.hi = d->clamp_hi;
        a.post_mul = d->post_mul;
        a.reduce_max_c = d->reduce_max_c;
        e = launch_cl_apply(a, L.cg, part, d->eps, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    if (L.recompute && conv2d_c8_recompute(g, x, out)) {
        C8Chain c8;
        c8.pre_mul = d->pre_mul;
        c8.part = ws_at<float4>(workspace, L.c8part);
        c8.xstats = ws_at<unsigned long long>(workspace, L.c8stats);
        c8.eps = d->eps;
        c8.run = RunningStats{d->running_mean, d->running_var, d->momentum};
        c8.flags = ws_at<uint32_t>(workspace, 0);
        c8.gamma = d->gamma;
        c8.beta = d->beta;
        c8.out_scale = d->out_scale;
        c8.clamp = d->clamp;
        c8.lo = d->clamp_lo;
        c8.hi = d->clamp_hi;
        c8.post_mul = d->post_mul;
        const hipError_t e = launch_conv2d_c8_bn_chain(g, x, w, b, out, c8, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    if (L.resident) {
        if (!aligned(out, 16))
            return fail(NR_ERR_MISALIGNED, "%s: out must be 16-byte aligned for this shape", fn);
        hipError_t e = launch_conv_k3(g, x, w, b, out, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        ResidentArgs a = resident_args(out, out, g.N, g.Cout, g.SP, batch, L.P, d->eps, d->gamma,
                                       d->beta, d->out_scale, nullptr, nullptr, workspace, L.exch,
                                       L.P > 1);
        a.pre_mul = d->pre_mul;
        a.clamp = d->clamp;
        a.lo = d->clamp_lo;
        a.hi = d->clamp_hi;
        a.post_mul = d->post_mul;
        a.running_mean = d->running_mean;
        a.running_var = d->running_var;
        a.momentum = d->momentum;
        e = launch_resident(resident_cfg(L.cfg_idx), a, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    if (L.ring_J > 0 ? g.N * g.Cout > 0x7fffffffLL : L.sg.slices * L.sg.chunks > 0x7fffffffLL)
        return fail(NR_ERR_UNSUPPORTED, "%s: too many statistics chunks for one launch", fn);

    float* c = ws_at<float>(workspace, L.cbuf);
    GroupStat* stats = ws_at<GroupStat>(workspace, L.stats);
    const RingStats rs{ws_at<float4>(workspace, L.partials), d->pre_mul, L.ring_J};
    ChainArgs a;
    a.c = c;
    a.out = out;
    a.N = g.N;
    a.Cout = g.Cout;
    a.SP = g.SP;
    a.batch = batch;
    a.stats = stats;
    a.pre_mul = d->pre_mul;
    a.gamma = d->gamma;
    a.beta = d->beta;
    a.out_scale = d->out_scale;
    a.clamp = d->clamp;
    a.lo = d->clamp_lo;
    a.hi = d->clamp_hi;
    a.post_mul = d->post_mul;
    a.reduce_max_c = d->reduce_max_c;
    hipError_t e;
    if (L.ring_J > 0) {
        e = launch_conv_k3_stats(g, x, w, b, c, rs, stream);
        if (e == hipSuccess && chain_apply_slots_ok(a)) {
            // the epilogue merges the slots itself
            e = launch_chain_apply_slots(a, rs, d->eps, stream);
            if (e != hipSuccess) return hip_fail(e, fn);
            return NR_OK;
        }
        if (e == hipSuccess) e = launch_ring_stats_merge(g, rs, d->eps, stats, stream);
    } else {
        e = launch_conv_k3(g, x, w, b, c, stream);
        if (e == hipSuccess)
            e = launch_split_stats(L.sg, c, d->pre_mul, ws_at<float2>(workspace, L.partials), d->eps,
                                   stats, nullptr, nullptr,
                                   RunningStats{d->running_mean, d->running_var, d->momentum},
                                   stream, true);
    }
    if (e != hipSuccess) return hip_fail(e, fn);
    e = launch_chain_apply(a, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return NR_OK;
}

// Eval-mode conv + batch norm: workspace = folded weights then folded bias.
size_t bn_eval_layout(const ConvGeom& g, size_t* off_b)
{
    const int64_t K = g.Cin * (g.dims == 3 ? 27 : 9);
    size_t off = kHeaderBytes;
    off = align_up(off + (size_t)(g.Cout * K) * sizeof(float), kWsAlign);
    *off_b = off;
    return align_up(off + (size_t)g.Cout * sizeof(float), kWsAlign);
}

nr_status check_eval_desc(const nr_conv_norm_desc* d, ConvGeom* g, const char* fn)
{
    nr_status s = check_desc(d, g, fn);
    if (s != NR_OK) return s;
    if (d->norm != NR_NORM_BATCH_TRAIN)
        return fail(NR_ERR_INVALID_ARG, "%s: norm must be NR_NORM_BATCH_TRAIN", fn);
    if (d->pre_mul || d->post_mul || d->clamp || d->reduce_max_c || d->running_mean || d->running_var)
        return fail(NR_ERR_UNSUPPORTED,
                    "%s: eval mode supports gamma, beta and out_scale only (no pre/post multiply, "
                    "clamp, max over channels or running-statistics update)", fn);
    return NR_OK;
}

__attribute__((visibility("default"))) size_t conv_bn_eval_workspace_size(const nr_conv_norm_desc* d)
{
    ConvGeom g;
    if (check_eval_desc(d, &g, "conv_bn_eval_workspace_size") != NR_OK) return 0;
    size_t ob;
    return bn_eval_layout(g, &ob);
}

__attribute__((visibility("default"))) nr_status conv_bn_eval_forward(
    const nr_conv_norm_desc* d, const float* x, const float* w, const float* b,
    const float* running_mean, const float* running_var, float* out, void* workspace,
    size_t workspace_bytes, hipStream_t stream)
{
    static const char* fn = "conv_bn_eval_forward";
    ConvGeom g;
    nr_status s = check_eval_desc(d, &g, fn);
    if (s != NR_OK) return s;
    if (g.N == 0) return NR_OK;  // empty batch
    if (!x || !w || !out || !running_mean || !running_var)
        return fail(NR_ERR_INVALID_ARG, "%s: x, w, running_mean, running_var and out must be non-NULL", fn);
    if (!aligned(x, 4) || !aligned(w, 4) || !aligned(out, 4) || (b && !aligned(b, 4)) ||
        !aligned(running_mean, 4) || !aligned(running_var, 4))
        return fail(NR_ERR_MISALIGNED, "%s: tensors must be 4-byte aligned", fn);
    size_t off_b;
    const size_t need = bn_eval_layout(g, &off_b);
    if ((s = check_workspace(workspace, workspace_bytes, need, fn)) != NR_OK) return s;
    // the matrix producers fold the statistics into W and b as they stage them
    if (conv_k3_eval_direct_ok(g, x, out)) {
        const ConvFold fold{running_mean, running_var, d->gamma, d->beta, d->eps, d->out_scale};
        const hipError_t e = launch_conv_k3_eval(g, x, w, b, fold, out, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return NR_OK;
    }
    float* wf = ws_at<float>(workspace, kHeaderBytes);
    float* bf = ws_at<float>(workspace, off_b);
    hipError_t e = launch_fold_bn_eval(g, w, b, running_mean, running_var, d->gamma, d->beta,
                                       d->eps, d->out_scale, wf, bf, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    e = launch_conv_k3(g, x, wf, bf, out, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return NR_OK;
}

__attribute__((visibility("default"))) nr_status nr_workspace_clear(void* workspace, size_t bytes,
                                                                    hipStream_t stream)
{
    if (!workspace) return fail(NR_ERR_INVALID_ARG, "nr_workspace_clear: workspace is NULL");
    if (bytes == 0) return NR_OK;
    const hipError_t e = launch_fill_zero(workspace, bytes, stream);
    if (e != hipSuccess) return hip_fail(e, "nr_workspace_clear");
    return NR_OK;
}

__attribute__((visibility("default"))) nr_status nr_workspace_check(void* workspace, size_t bytes,
                                                                    hipStream_t stream,
                                                                    uint32_t* flags_out)
{
    static const char* fn = "nr_workspace_check";
    if (!workspace || !flags_out) return fail(NR_ERR_INVALID_ARG, "%s: NULL argument", fn);
    if (bytes < kHeaderBytes) return fail(NR_ERR_WORKSPACE, "%s: workspace smaller than its header", fn);
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    uint32_t flags = 0, zero = 0;
    e = hipMemcpy(&flags, workspace, sizeof(flags), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (flags) {
        e = hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    *flags_out = flags;
    return NR_OK;
}

__attribute__((visibility("default"))) nr_status nr_stream_copy(const float* src, float* dst, int64_t n,
                                                                hipStream_t stream)
{
    if (!src || !dst || n < 0) return fail(NR_ERR_INVALID_ARG, "nr_stream_copy: bad arguments");
    if (!aligned(src, 4) || !aligned(dst, 4)) return fail(NR_ERR_MISALIGNED, "nr_stream_copy: misaligned");
    if (ranges_partially_overlap(src, dst, n) || (src == dst && n > 0))
        return fail(NR_ERR_INVALID_ARG, "nr_stream_copy: src and dst overlap");
    const hipError_t e = launch_stream_copy(src, dst, n, stream);
    if (e != hipSuccess) return hip_fail(e, "nr_stream_copy");
    return NR_OK;
}

__attribute__((visibility("default"))) nr_status nr_stream_copy_ws(const float* src, float* dst,
                                                                   int64_t n, void* workspace,
                                                                   size_t workspace_bytes,
                                                                   hipStream_t stream)
{
    static const char* fn = "nr_stream_copy_ws";
    if (!src || !dst || n < 0) return fail(NR_ERR_INVALID_ARG, "%s: bad arguments", fn);
    if (!aligned(src, 4) || !aligned(dst, 4)) return fail(NR_ERR_MISALIGNED, "%s: misaligned", fn);
    if (ranges_partially_overlap(src, dst, n) || (src == dst && n > 0))
        return fail(NR_ERR_INVALID_ARG, "%s: src and dst overlap", fn);
    if (!workspace || workspace_bytes < 256 || !aligned(workspace, 256))
        return fail(NR_ERR_WORKSPACE, "%s: needs a 256-byte aligned workspace of >= 256 bytes", fn);
    const bool vec = aligned(src, 16) && aligned(dst, 16) && n % 4 == 0;
    const hipError_t e = vec ? launch_stream_copy_persistent(src, dst, n, workspace, stream)
                             : launch_stream_copy(src, dst, n, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return NR_OK;
}

}  // extern "C"
