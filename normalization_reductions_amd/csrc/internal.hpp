// internal.hpp -- host-side interfaces between the C ABI layer (abi.cpp) and the kernel
// launchers (*.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "normred.h"
#include "resident.hpp"

namespace nr {

// Records the message nr_last_error() returns on this thread and returns s (abi.cpp).
nr_status set_error(nr_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// ---------------------------------------------------------------------------------------------
// Workspace regions (byte offsets inside the caller's workspace; every region 256-B aligned).
// ---------------------------------------------------------------------------------------------
constexpr size_t kWsAlign = 256;
constexpr size_t kHeaderBytes = 256;     // uint32 flags at offset 0

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Read-once normalization: see resident.hpp.

// Read-once instance normalization of slices with S % 4 != 0 (flat_norm.hip): one workgroup
// per slice (or per group of 4 to 32 lanes for short slices), x and y 16-byte aligned,
// S <= flat_norm_max_len(), slices <= 2^31 - 1, slices * S >= 4.
int64_t flat_norm_max_len();
// Read-once training-mode batch norm of slices with S % 4 != 0 (flat_norm.hip): one workgroup
// per channel when the channel's N slices fit it and all C workgroups are resident at once
// (flat_bn_fits); x and y 16-byte aligned, C <= 2^31 - 1, N * C * S >= 4.
bool flat_bn_fits(int64_t N, int64_t C, int64_t S);
hipError_t launch_flat_bn(const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps,
                          const float* gamma, const float* beta, float out_scale,
                          float* save_mean, float* save_invstd, float* running_mean,
                          float* running_var, float momentum, hipStream_t stream);
hipError_t launch_flat_norm(const float* x, float* y, int64_t slices, int64_t C, int64_t S,
                            float eps, const float* gamma, const float* beta, float* save_mean,
                            float* save_invstd, hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Streaming split path: partial statistics per (slice, chunk) -> fixed-order merge per group
// -> apply. Groups are slices (instance norm) or channels (batch norm).
// ---------------------------------------------------------------------------------------------
struct SplitGeom {
    int64_t S = 0;        // slice length
    int64_t slices = 0;   // N*C
    int64_t C = 0;        // channels (slice's channel = slice % C)
    int64_t chunk = 0;    // elements per chunk (multiple of 4 * block), last chunk may be shorter
    int64_t chunks = 0;   // ceil(S / chunk)
    bool batch = false;   // true: group = channel over all n; false: group = slice
    bool vec = false;     // 16-B path (aligned pointers and S % 4 == 0)
};

struct GroupStat {    // per group, written by the merge step
    float pivot;      // the value the statistics are taken relative to
    float mean_d;     // mean - pivot
    float rstd;       // 1 / sqrt(var + eps)
    float pad;
};

SplitGeom split_geometry(int64_t N, int64_t C, int64_t S, bool batch, bool vec);


struct RunningStats {      // optional in-place running-statistics update (batch groups)
    float* mean = nullptr;
    float* var = nullptr;
    float momentum = 0.f;
};

// Group statistics: partials per (slice, chunk), then the fixed-order merge; instance groups of
// one chunk write their statistics directly. cached: plain loads (a chain's conv output, read
// again by the epilogue right after); otherwise streaming loads.
hipError_t launch_split_stats(const SplitGeom& g, const float* x, const float* pre_mul,
                              float2* partials, float eps, GroupStat* stats, float* save_mean,
                              float* save_invstd, RunningStats run, hipStream_t stream,
                              bool cached = false);
hipError_t launch_split_apply(const SplitGeom& g, const float* x, float* y,
                              const GroupStat* stats, const float* gamma, const float* beta,
                              float out_scale, hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Convolution producer and the chain epilogue.
// ---------------------------------------------------------------------------------------------
struct ConvGeom {
    int dims;                  // 2 or 3
    int64_t N, Cin, Cout;
    int64_t D, H, W;           // input extent (D = 1 for 2-D)
    int64_t OD, OH, OW, SP;    // output extent, SP = OD*OH*OW
    int cl = 0;                // channels last: x [N, D, H, W, Cin], output [N, SP, Cout]
};

// Geometry of the persistent conv producer: the output as N * OO outer slices (rows in 2-D,
// depth planes in 3-D) of T tiles of 16 positions each.
struct ConvRing {
    int OO;         // outer output slices per batch item (OH or OD)
    int outer_in;   // H or D
    int inner_in;   // W or H*W: floats per input slice of one channel
    int inner_out;  // OW or OH*OW: positions per output slice
    int T;          // tiles per output slice (including the alignment shift)
    int vec_in;     // 16-byte input loads
    int vec_out;    // 16-byte output stores (aligned groups of 4 positions)
};

// Eval-mode batch norm folded into a conv producer as it stages W: output channel k's weights
// scaled by gamma[k] / sqrt(rv[k] + eps) * scale, its bias to ((b[k] - rm[k]) * that + beta[k])
// * scale (rv NULL: no fold).
struct ConvFold {
    const float* rm;
    const float* rv;
    const float* gamma;  // or NULL
    const float* beta;   // or NULL
    float eps, scale;
};

// Instance-norm statistics the ring producer takes of its own output: per batch item n, J slots
// of partials per channel, merged in slot order by the reader.
struct RingStats {
    float4* part;          // [N][J][Cout]: (count, mean, M2, 0) of pre_mul * c
    const float* pre_mul;  // [Cout] or NULL
    int64_t J;             // slots per batch item
};

// Epilogue and statistics arguments of the 2-D C_in 8 -> C_out 64 matrix producer when it runs
// a batch-norm chain by recomputation (statistics pass, merge, apply pass).
struct C8Chain {
    const float* pre_mul = nullptr;
    float4* part = nullptr;         // [C_out][nparts] (count, mean, M2, -), by the statistics pass
    // [C_out][2] tagged words (mean, rstd): zeroed by the statistics pass; the apply pass's
    // first workgroups merge the partials of one channel each and publish them here, and every
    // workgroup reads its channels' words before its first epilogue
    unsigned long long* xstats = nullptr;
    int nparts = 0;                 // partials per channel (the statistics pass's workgroups)
    float eps = 0.f;
    RunningStats run;               // optional running-statistics update (by the merging workgroups)
    uint32_t* flags = nullptr;      // sticky error word: a wait for the published words gave up
    uint32_t wait_tag = 1, spin_limit = 0;  // the tag the readers accept and their polling bound:
                                            // set by the launcher (see launch_resident)
    const float* gamma = nullptr;
    const float* beta = nullptr;
    float out_scale = 1.f;
    int clamp = 0;
    float lo = 0.f, hi = 0.f;
    const float* post_mul = nullptr;
    // eval mode folded into the conv (kC8Conv): when fold_rv is set, W and b are scaled per output
    // channel k by gamma[k] / sqrt(fold_rv[k] + eps) * out_scale, b shifted by fold_rm[k] and beta
    const float* fold_rm = nullptr;
    const float* fold_rv = nullptr;
};

// The 2-D C_in 8 -> C_out 64, W = 64 shapes of the matrix producer (pointer alignment aside):
// even output heights, int32 offsets within a batch item.
bool conv2d_c8_shape(const ConvGeom& g);
// Workgroups of its statistics pass (the number of partials per channel); at most kC8MaxGrid.
constexpr int64_t kC8MaxGrid = 4096;
int64_t conv2d_c8_stats_grid(const ConvGeom& g);
// An upper bound of conv2d_c8_stats_grid on any device (one workgroup per box at most), for
// sizing the partials before a device is known.
int64_t conv2d_c8_grid_bound(const ConvGeom& g);
// Whether a batch-norm chain of this shape and these pointers runs by recomputation (the
// bf16x6 producer is not overridden for comparisons).
bool conv2d_c8_recompute(const ConvGeom& g, const void* x, const void* out);
// Batch-norm chain by recomputation: statistics pass into e.part, fixed-order merge into
// stats (and the running statistics), then the conv again with the chain epilogue into out.
// Needs conv2d_c8_shape(g) and 16-byte aligned x and out.
// Eval-mode batch norm folded into the matrix producers (the 2-D 64-wide one and the ring) as
// they stage W, with no fold launch; false where no matrix producer takes the call (the caller
// then folds W and b and calls launch_conv_k3).
bool conv_k3_eval_direct_ok(const ConvGeom& g, const void* x, const void* out);
hipError_t launch_conv_k3_eval(const ConvGeom& g, const float* x, const float* w, const float* b,
                               const ConvFold& fold, float* out, hipStream_t stream);
hipError_t launch_conv2d_c8_bn_chain(const ConvGeom& g, const float* x, const float* w,
                                     const float* b, float* out, C8Chain e, hipStream_t stream);
hipError_t launch_conv_k3(const ConvGeom& g, const float* x, const float* w, const float* b,
                          float* c, hipStream_t stream);
// Slots per batch item of the ring producer's own statistics for this shape, for any pointer
// alignment; 0 when the ring producer does not run the shape.
int64_t ring_stats_slots(const ConvGeom& g);
// The conv of launch_conv_k3 through the ring producer, which also writes the instance-norm
// partials rs (rs.J == ring_stats_slots(g) > 0).
hipError_t launch_conv_k3_stats(const ConvGeom& g, const float* x, const float* w, const float* b,
                                float* c, RingStats rs, hipStream_t stream);
// Group statistics per (n, k) from those partials (slot order), for the planar chain epilogue.
hipError_t launch_ring_stats_merge(const ConvGeom& g, const RingStats& rs, float eps,
                                   GroupStat* stats, hipStream_t stream);

// Eval-mode batch norm folded into conv weights: wf [Cout][Cin*k^dims], bf [Cout].
hipError_t launch_fold_bn_eval(const ConvGeom& g, const float* w, const float* b, const float* rm,
                               const float* rv, const float* gamma, const float* beta, float eps,
                               float scale, float* wf, float* bf, hipStream_t stream);

struct ChainArgs {
    const float* c;        // [N, Cout, SP] conv output
    float* out;            // [N, SP] (max over channels) or [N, Cout, SP]
    int64_t N, Cout, SP;
    bool batch;            // statistics per channel (true) or per (n, k) (false)
    const GroupStat* stats;
    const float* pre_mul;
    const float* gamma;
    const float* beta;
    float out_scale;
    int clamp;
    float lo, hi;
    const float* post_mul;
    int reduce_max_c;
};

hipError_t launch_chain_apply(const ChainArgs& a, hipStream_t stream);
// The same epilogue for instance norm with the statistics still in the ring producer's slots
// (each workgroup merges its item's slots); needs chain_apply_slots_ok(a).
bool chain_apply_slots_ok(const ChainArgs& a);
hipError_t launch_chain_apply_slots(const ChainArgs& a, const RingStats& rs, float eps,
                                   hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Channels-last chain: c [N, SP, C] (C contiguous). A group is (n, k) (instance) or k (batch);
// its values are C apart. Partials per (n, chunk of positions, k), merged in fixed order.
// ---------------------------------------------------------------------------------------------
struct ClGeom {
    int64_t N, C, SP;
    int64_t chunk;    // positions per partial
    int64_t chunks;   // partials per batch item: ceil(SP / chunk)
    bool batch;
};
ClGeom cl_geometry(int64_t N, int64_t C, int64_t SP, bool batch);
size_t cl_partials_bytes(const ClGeom& g);  // float4 per (n, chunk, k)
// Partials of every (n, chunk, k); for batch norm also their merge into stats (and the running
// statistics). Instance norm leaves the merge to launch_cl_apply.
hipError_t launch_cl_stats(const ClGeom& g, const float* c, const float* pre_mul, float4* partials,
                           float eps, GroupStat* stats, RunningStats run, hipStream_t stream);
// ChainArgs as for the planar chain, with c and (without the max) out in [N, SP, C] layout.
// Batch norm reads a.stats; instance norm merges the partials of launch_cl_stats itself.
hipError_t launch_cl_apply(const ChainArgs& a, const ClGeom& g, const float4* partials, float eps,
                           hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Utilities.
// ---------------------------------------------------------------------------------------------
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_stream_copy(const float* src, float* dst, int64_t n, hipStream_t stream);
// Persistent copy (src, dst 16-byte aligned, n % 4 == 0); counter: 4 device bytes it zeroes.
hipError_t launch_stream_copy_persistent(const float* src, float* dst, int64_t n, void* counter,
                                         hipStream_t stream);

}  // namespace nr
