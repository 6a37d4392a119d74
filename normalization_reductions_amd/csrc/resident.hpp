// resident.hpp -- host/device interface of the read-once normalization kernels
// (resident_norm.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nr {

constexpr int kMaxParts = 32;  // parts per statistics group in the read-once kernels

// Read-once ("resident") normalization: each statistics group (one slice for instance norm, the
// N slices of a channel for batch norm) split over P workgroups that run concurrently, each holding its
// part in registers.
struct ResidentCfg {
    int block;       // threads per workgroup
    int vec;         // float4 registers per thread (per buffer)
    int part_len;    // values per part = block * 4 * vec
    bool pipelined;  // false: one workgroup per group (P == 1); true: persistent, P > 1
    bool grouped;    // groups span several slices (batch norm)
    bool chain;      // pre-multiplier, clamp and post-multiplier in the epilogue
};

// The configurations compiled into the library.
int resident_cfg_count();
ResidentCfg resident_cfg(int i);

struct ResidentArgs {
    const float* x;
    float* y;             // may equal x
    int64_t S;            // slice length; S % 4 == 0, x and y 16-B aligned
    int64_t C;            // channels
    int64_t groups;       // N*C (instance) or C (batch)
    int64_t L;            // values per group: S (instance) or N*S (batch); < 2^21 when grouped
    uint64_t div_magic;   // ceil(2^42 / S): v / S for v < 2^21 (grouped kernels)
    int32_t batch;        // 1: group g = channel g over all n; 0: group g = slice g
    int32_t P;            // parts per group, 1..kMaxParts
    float eps;
    const float* gamma;   // [C] or NULL
    const float* beta;    // [C] or NULL
    float out_scale;
    const float* pre_mul;   // chain kernels: [C] or NULL
    int32_t clamp;          // chain kernels
    float lo, hi;
    const float* post_mul;  // chain kernels: [C] or NULL
    float* save_mean;       // [groups] or NULL
    float* save_invstd;     // [groups] or NULL
    float* running_mean;    // [groups] or NULL: updated in place (batch groups)
    float* running_var;     // [groups] or NULL (unbiased batch variance blended in)
    float momentum;
    uint32_t* counter;           // next unit to take; followed (256 B on) by the slots
    unsigned long long* slots;   // [groups][P][2] tagged exchange words
    uint32_t* flags;             // sticky error word
    // set by launch_resident: the tag an exchange wait accepts and its polling bound (the tag
    // the parts publish and kSpinLimit, except under the give-up test switch)
    uint32_t wait_tag;
    uint32_t spin_limit;
};

uint64_t resident_div_magic(int64_t S);

// Bytes a launch with P parts uses at `counter` (counter, then slots), zero-filled by
// launch_resident before every launch.
constexpr size_t kCounterBytes = 256;
inline size_t resident_ws_bytes(int64_t groups, int P)
{
    return P > 1 ? kCounterBytes + (size_t)groups * (size_t)P * 2 * sizeof(unsigned long long) : 0;
}

// Persistent grid of the pipelined kernel: CUs x min(occupancy, workgroups per CU wanted)
// (0 if the configuration is unknown).
int resident_max_grid(const ResidentCfg& cfg);
hipError_t launch_resident(const ResidentCfg& cfg, const ResidentArgs& a, hipStream_t stream);

}  // namespace nr
