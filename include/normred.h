/*
 * normred.h -- C ABI of the per-slice normalization library (libnormred.so), MI355X / gfx950.
 *
 * Three operations, as the source pages state them (pages of the "POPCORNBENCH / Kimi-K2.6"
 * kernel-task traces):
 *   IN2d page -- task l1_p34: InstanceNorm2d on x[112,64,512,512];
 *   BN page   -- task l2_p73: Conv2d(8->64,k=3) -> BatchNorm2d(64) -> x2.0;
 *   IN3d page -- task l2_p79: Conv3d(3->16,k=3) -> xmultiplier -> InstanceNorm3d -> clamp ->
 *                xmultiplier -> max over channels.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major fp32 in DEVICE memory. The caller allocates and owns every
 *     buffer (inputs, outputs, workspace); the library never allocates, frees or synchronizes
 *     inside these calls.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call returns at once.
 *   - Arguments are validated on the host before anything is enqueued; a rejected call returns
 *     a non-zero nr_status, enqueues nothing and leaves every buffer untouched. The message for
 *     the most recent failure on the calling thread is nr_last_error().
 *   - NR_ERR_HIP reports a HIP runtime error raised while enqueueing. Faults inside kernels
 *     surface at the caller's next synchronization, as with any HIP launch.
 *   - Results are deterministic: the same inputs and shapes give bit-identical outputs on
 *     every run (fixed reduction order; no floating-point atomics).
 *   - Workspace: a device buffer (256-byte aligned) of at least the size the matching
 *     *_workspace_size query returns. Its contents need no initialization and carry nothing
 *     from one call to the next, except the sticky error word that nr_workspace_check reads
 *     (zero the buffer once, e.g. with nr_workspace_clear, to use that check). Calls that share
 *     a workspace must be ordered (same stream, or synchronized): concurrent calls on one
 *     workspace race.
 */
#ifndef NORMRED_H
#define NORMRED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nr_status {
    NR_OK = 0,
    NR_ERR_INVALID_ARG = 1, /* null pointer, non-positive or overflowing size, bad option */
    NR_ERR_MISALIGNED = 2,  /* a pointer misaligned for its element type (4 bytes for fp32) */
    NR_ERR_UNSUPPORTED = 3, /* a valid request this library does not implement (e.g. ksize != 3) */
    NR_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the size query */
    NR_ERR_HIP = 5          /* HIP runtime error while enqueueing */
} nr_status;

/* Message for the last non-OK status returned on this thread ("" if none). Never NULL. */
const char* nr_last_error(void);

/* Library version string, e.g. "normred 0.1.0 gfx950". */
const char* nr_version(void);

/* ------------------------------------------------------------------------------------------
 * Instance normalization.
 *
 * IN2d page, statement of the op (and IN3d page, its InstanceNorm3d reading): for every
 * (n, c) slice of S = H*W (or D*H*W) elements, mean and BIASED variance over the slice, then
 *     y = (x - mean) / sqrt(var + eps)              (affine = False, the pages' default)
 * and, when gamma/beta are given, y = that * gamma[c] + beta[c].
 *
 * x, y       : [N, C, S] fp32 device buffers. y may equal x (in place); partial overlap is
 *              rejected (NR_ERR_INVALID_ARG).
 * N, C, S    : sizes; S >= 1, N >= 0, C >= 0. N*C == 0 is an empty batch: NR_OK, nothing
 *              enqueued, and every pointer (x, y, workspace, ...) may be NULL. N*C*S*4 must
 *              fit in int64.
 * eps        : added to the variance inside the square root (the pages use 1e-5); >= 0.
 * gamma,beta : [C] device buffers, or both NULL (affine = False). One without the other is
 *              rejected.
 * save_mean, save_invstd : [N*C] device outputs, or NULL: the slice mean and 1/sqrt(var+eps).
 * workspace  : device buffer of >= inorm_workspace_size(N, C, S) bytes (see conventions).
 * ------------------------------------------------------------------------------------------ */
size_t inorm_workspace_size(int64_t N, int64_t C, int64_t S);

nr_status inorm_forward(const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps,
                        const float* gamma, const float* beta, float* save_mean,
                        float* save_invstd, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Kernel variants for inorm_forward_ex (benchmarks and tests; inorm_forward = AUTO). */
#define NR_VARIANT_AUTO 0     /* the library's choice for the shape */
#define NR_VARIANT_RESIDENT 1 /* read-once: each slice held in registers, split over 1..32
                                 concurrent workgroups that exchange partial statistics; a
                                 slice with S % 4 != 0 (S <= 65,530) or S < 1024 is held by
                                 one workgroup sized to it. Needs 16-byte aligned x and y */
#define NR_VARIANT_SPLIT 2    /* streaming two-pass: partial statistics per chunk, a fixed-order
                                 merge, then a normalize pass (reads x twice) */

/* As inorm_forward, with an explicit variant. A variant that cannot run this shape (e.g.
 * RESIDENT with a slice beyond 32 parts, or unaligned data) returns NR_ERR_UNSUPPORTED. */
nr_status inorm_forward_ex(const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps,
                           const float* gamma, const float* beta, float* save_mean,
                           float* save_invstd, void* workspace, size_t workspace_bytes,
                           int variant, hipStream_t stream);

/* For callers that cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): inorm_forward with the library's own workspace, a
 * device array of 8 MiB (8388608 bytes) that the library holds on every GPU it runs on until
 * the process ends. Arguments as inorm_forward. Shapes whose inorm_workspace_size exceeds
 * 8 MiB are rejected with NR_ERR_WORKSPACE (x[112,64,512,512] needs 3.7 MiB). Nothing is
 * allocated or freed: the array's address is looked up once per device, on the first call
 * with that device current. Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (two streams, or threads without ordering) race; order them. */
nr_status inorm_forward_noalloc(const float* x, float* y, int64_t N, int64_t C, int64_t S,
                                float eps, const float* gamma, const float* beta,
                                float* save_mean, float* save_invstd, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Training-mode batch normalization, then a scale.
 *
 * BN page, opening analysis: in training mode the output uses the batch statistics -- per
 * channel c, mean and BIASED variance over all (n, spatial) -- and
 *     y = ((x - mean_c) / sqrt(var_c + eps) * gamma[c] + beta[c]) * out_scale
 * (the page's model multiplies by scaling_factor = 2.0 after the norm). Running statistics
 * are neither read nor written.
 *
 * x, y       : [N, C, S] fp32 device buffers; y may equal x.
 * N, C, S    : N >= 1 and S >= 1 (statistics over nothing are undefined); C >= 0 (C == 0 is
 *              a no-op that accepts NULL pointers).
 * gamma,beta : [C] device buffers, or both NULL (identity affine).
 * out_scale  : final multiplier (1.0f for plain batch norm).
 * save_mean, save_invstd : [C] device outputs, or NULL.
 * workspace  : >= bn_train_workspace_size(N, C, S) bytes.
 * ------------------------------------------------------------------------------------------ */
size_t bn_train_workspace_size(int64_t N, int64_t C, int64_t S);

nr_status bn_train_forward(const float* x, float* y, int64_t N, int64_t C, int64_t S, float eps,
                           const float* gamma, const float* beta, float out_scale,
                           float* save_mean, float* save_invstd, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* As bn_train_forward, and also blends the batch statistics into running statistics in
 * place -- BN page, opening analysis: a training step moves running_mean and running_var
 * toward the batch mean and the UNBIASED batch variance (biased * n / (n - 1), n = N*S) with
 *     running = (1 - momentum) * running + momentum * batch        (the pages use 0.1).
 * running_mean, running_var: [C] device buffers, both given or both NULL (no update).
 * momentum: in [0, 1]. An update needs N*S >= 2 (NR_ERR_INVALID_ARG otherwise). */
nr_status bn_train_forward_ex(const float* x, float* y, int64_t N, int64_t C, int64_t S,
                              float eps, const float* gamma, const float* beta, float out_scale,
                              float* save_mean, float* save_invstd, float momentum,
                              float* running_mean, float* running_var, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Convolution (k = 3, stride 1, no padding, with bias) -> normalization -> epilogue.
 *
 * The step order covers both model pages:
 *   c  = conv(x, w) + b        cross-correlation, no kernel flip (BN page, its direct-conv
 *                              indexing; IN3d page: output extent = input extent - 2)
 *   s  = c * pre_mul[k]        (IN3d page: first multiply by the [C,1,1,1] multiplier)
 *   z  = (s - mean) / sqrt(var + eps)
 *        NR_NORM_BATCH_TRAIN: statistics per channel k over (n, spatial)   (BN page)
 *        NR_NORM_INSTANCE   : statistics per (n, k) over spatial           (IN3d page)
 *   z  = z * gamma[k] + beta[k]  (BN page: affine batch norm)
 *   z  = z * out_scale           (BN page: x scaling_factor)
 *   z  = min(max(z, lo), hi)     (IN3d page: clamp, in its min(max()) order), if clamp
 *   u  = z * post_mul[k]         (IN3d page: second multiply)
 *   out = max over k of u        if reduce_max_c (IN3d page: max over dim 1, values only)
 *       = u                      otherwise
 *
 * Shapes: x [N, C_in, (D,) H, W]; w [C_out, C_in, (3,) 3, 3]; b [C_out] or NULL;
 * out [N, (D-2,) H-2, W-2] if reduce_max_c else [N, C_out, (D-2,) H-2, W-2].
 * spatial_dims is 2 (D ignored) or 3. Every optional [C_out] pointer may be NULL. N == 0 is an
 * empty batch (NR_OK, nothing enqueued; x, w, out and workspace may be NULL).
 * When reduce_max_c == 0 and the output's spatial size is a multiple of 4 (and the statistics
 * groups fit the read-once kernels), the conv writes straight into `out`, which is then
 * normalized in place: `out` must be 16-byte aligned (else NR_ERR_MISALIGNED) and the workspace
 * holds only exchange slots. Otherwise the conv output is staged in the workspace.
 * Batch norm on the 2-D shape C_in 8 -> C_out 64 with in_w = 64 and an even output height (the
 * BN page's model) runs the conv twice instead, when x and out are 16-byte aligned: a
 * statistics pass, then the conv again with the epilogue, so that c never goes to memory (the
 * workspace holds per-workgroup partial statistics, at most 4 MiB); with other pointers the
 * in-place plan above runs.
 * Instance norm on the shapes C_in 3 -> C_out 16 (3-D, the IN3d page's model) and C_in 8 ->
 * C_out 64 (2-D, other than the shape above), when the conv output is staged or channels last:
 * the conv producer takes the statistics of its own output (the workspace holds N x J x C_out
 * partials of 16 bytes, J a few per batch item), so no pass re-reads the conv output for them.
 * Precision: the conv is fp32-accurate. On that 2-D shape its products come from exact
 * three-part bf16 splits of x and w (six partial products; each part left out is below
 * 2^-24 |x w|); the statistics pass forms the same products as the pass that normalizes, so a
 * channel of zero variance (e.g. a constant input) gives exactly beta * out_scale.
 *
 * Channels last (channels_last = 1; IN3d page, its note on an (N, spatial, C) layout that makes
 * the max over channels contiguous): x is [N, (D,) H, W, C_in] and out is
 * [N, (D-2,) H-2, W-2, C_out], or [N, (D-2,) H-2, W-2] with reduce_max_c; w keeps its layout.
 * The arithmetic and the step order are the same. C_out <= 256 (else NR_ERR_UNSUPPORTED). The
 * conv output is staged in the workspace when reduce_max_c, else written to `out` and normalized
 * in place; the statistics come from the producer as above, or from a pass over it. No
 * alignment is required.
 * ------------------------------------------------------------------------------------------ */
#define NR_NORM_BATCH_TRAIN 1
#define NR_NORM_INSTANCE 2

typedef struct nr_conv_norm_desc {
    int32_t spatial_dims;        /* 2 or 3 */
    int32_t ksize;               /* must be 3, else NR_ERR_UNSUPPORTED */
    int64_t N, C_in, C_out;      /* >= 1 each */
    int64_t in_d, in_h, in_w;    /* input extent; in_d ignored when spatial_dims == 2; >= 3 */
    int32_t norm;                /* NR_NORM_BATCH_TRAIN or NR_NORM_INSTANCE */
    float eps;                   /* >= 0 */
    const float* pre_mul;        /* [C_out] or NULL */
    const float* gamma;          /* [C_out] or NULL */
    const float* beta;           /* [C_out] or NULL */
    float out_scale;             /* 1.0f = none */
    int32_t clamp;               /* 0 or 1 */
    float clamp_lo, clamp_hi;    /* used when clamp = 1; lo <= hi */
    const float* post_mul;       /* [C_out] or NULL */
    int32_t reduce_max_c;        /* 0 or 1 */
    float momentum;              /* running-statistics update (NR_NORM_BATCH_TRAIN only), */
    float* running_mean;         /* as in bn_train_forward_ex: [C_out] each, both or neither */
    float* running_var;
    int32_t channels_last;       /* 0: x, out planar (N, C, spatial); 1: (N, spatial, C) */
} nr_conv_norm_desc;

/* 0 if the descriptor is invalid. */
size_t conv_norm_epilogue_workspace_size(const nr_conv_norm_desc* d);

nr_status conv_norm_epilogue_forward(const nr_conv_norm_desc* d, const float* x, const float* w,
                                     const float* b, float* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Convolution (k = 3, stride 1, no padding, with bias) -> eval-mode batch normalization with
 * running statistics -> x out_scale, folded into one conv pass.
 *
 * BN page, its eval-mode discussion: with running statistics the norm is a per-channel affine
 * map, so it folds into the conv: a_k = gamma[k] * out_scale / sqrt(running_var[k] + eps),
 * W'[k] = W[k] * a_k, b'[k] = ((b[k] - running_mean[k]) * gamma[k] / sqrt(running_var[k] + eps)
 * + beta[k]) * out_scale, then out = conv(x, W') + b'.
 *
 * d: shapes, eps, gamma, beta, out_scale are used; d->norm must be NR_NORM_BATCH_TRAIN (the
 *    batch-norm kind; no batch statistics are computed here); pre_mul, post_mul,
 *    clamp, reduce_max_c and the running-statistics update fields must be unset
 *    (NR_ERR_UNSUPPORTED otherwise).
 * running_mean, running_var: [C_out] device buffers (read only).
 * out: [N, C_out, (D-2,) H-2, W-2], or [N, (D-2,) H-2, W-2, C_out] with d->channels_last (x
 *    then [N, (D,) H, W, C_in]). workspace: >= conv_bn_eval_workspace_size(d) bytes (holds the
 *    folded weights; refilled by every call).
 * ------------------------------------------------------------------------------------------ */
size_t conv_bn_eval_workspace_size(const nr_conv_norm_desc* d);

nr_status conv_bn_eval_forward(const nr_conv_norm_desc* d, const float* x, const float* w,
                               const float* b, const float* running_mean,
                               const float* running_var, float* out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Workspace and measurement helpers.
 * ------------------------------------------------------------------------------------------ */

/* Zero-fill `bytes` of a workspace on `stream` with a fill kernel (no hipMemset, so it is
 * also safe inside a captured graph). */
nr_status nr_workspace_clear(void* workspace, size_t bytes, hipStream_t stream);

/* Reads the workspace's sticky error word (synchronizes `stream` first). *flags_out = 0 when
 * every exchange wait completed; bit 0 = a bounded wait gave up (results of that call are
 * invalid). Clears the word afterwards. */
nr_status nr_workspace_check(void* workspace, size_t bytes, hipStream_t stream, uint32_t* flags_out);

/* Plain streaming copy dst[i] = src[i], i < n, with 16-byte loads/stores: the HBM ceiling the
 * normalization kernels are compared against, and the calibration kernel for byte counters.
 * src/dst 16-byte aligned and n % 4 == 0 for the vector path; anything else takes a scalar
 * path. */
nr_status nr_stream_copy(const float* src, float* dst, int64_t n, hipStream_t stream);

/* The same copy in the fastest pattern measured on MI355X: one persistent workgroup per CU
 * taking 64 KiB units in order from a counter kept in `workspace` (>= 256 bytes, 256-byte
 * aligned; its first 4 bytes are zeroed on `stream` and then used). Vector path under the same
 * conditions as nr_stream_copy, which serves every other call. Calls sharing a workspace must
 * be ordered. */
nr_status nr_stream_copy_ws(const float* src, float* dst, int64_t n, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NORMRED_H */
