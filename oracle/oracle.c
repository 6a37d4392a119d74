/*
 * oracle.c -- plain, slow, fp64 CPU reference for the per-slice normalization path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg load this library. The HIP library never links, calls or includes anything from here,
 * and nothing here is shared with it.
 *
 * Every function is the plain mathematical definition written out:
 *   - inputs are fp32, widened to double on load;
 *   - sums are sequential fp64 loops; the variance is the two-pass textbook form
 *     (mean first, then the mean of squared deviations), biased (divide by the count);
 *   - results are rounded to fp32 exactly once, at the very end.
 * Loops follow the order in which the source pages state each operation. Threads only split
 * independent slices / channels / batch items; they never change the arithmetic of one result.
 *
 * Sources (pages of the "POPCORNBENCH / Kimi-K2.6" kernel-task traces):
 *   IN2d page  -- task l1_p34, InstanceNorm2d on x[112,64,512,512];
 *   BN page    -- task l2_p73, Conv2d(8->64,k=3) -> BatchNorm2d(64) -> x2.0;
 *   IN3d page  -- task l2_p79, Conv3d(3->16,k=3) -> xmultiplier -> InstanceNorm3d -> clamp
 *                 -> xmultiplier -> max over channels.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define OR_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------------------------ */
/* A tiny fork/join helper: run body(arg, lo, hi) over [0, n) split into contiguous ranges.   */
/* ------------------------------------------------------------------------------------------ */
typedef void (*range_fn)(void* arg, int64_t lo, int64_t hi);

typedef struct {
    range_fn fn;
    void* arg;
    int64_t lo, hi;
} range_job;

static void* range_trampoline(void* p)
{
    range_job* j = (range_job*)p;
    j->fn(j->arg, j->lo, j->hi);
    return NULL;
}

static int resolve_threads(int nthreads)
{
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void* arg)
{
    int t = resolve_threads(nthreads);
    if (t > 256) t = 256;
    if ((int64_t)t > n) t = (int)(n > 0 ? n : 1);
    if (t <= 1) {
        fn(arg, 0, n);
        return;
    }
    pthread_t tid[256];
    range_job jobs[256];
    int started = 0;
    for (int i = 0; i < t; ++i) {
        jobs[i].fn = fn;
        jobs[i].arg = arg;
        jobs[i].lo = n * i / t;
        jobs[i].hi = n * (i + 1) / t;
        if (pthread_create(&tid[i], NULL, range_trampoline, &jobs[i]) != 0) {
            /* could not start a thread: do this range on the calling thread instead */
            fn(arg, jobs[i].lo, jobs[i].hi);
            jobs[i].fn = NULL;
        } else {
            ++started;
        }
    }
    for (int i = 0; i < t; ++i)
        if (jobs[i].fn) pthread_join(tid[i], NULL);
    (void)started;
}

OR_API int or_default_threads(void) { return resolve_threads(0); }

/* ------------------------------------------------------------------------------------------ */
/* Instance normalization over one slice.                                                     */
/*                                                                                            */
/* IN2d page, statement of the op: for each (n, c) take the mean and the biased variance over */
/* the H*W elements, then y = (x - mean) / sqrt(var + eps) with eps = 1e-5, no affine by      */
/* default. IN3d page, its reading of InstanceNorm3d: the same over D*H*W. With affine        */
/* parameters, y is further multiplied by gamma[c] and shifted by beta[c].                    */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    const float* x;
    float* y;
    int64_t S, C;
    double eps;
    const float* gamma;
    const float* beta;
    double* mean_out;
    double* var_out;
} in_args;

static void in_range(void* p, int64_t lo, int64_t hi)
{
    const in_args* a = (const in_args*)p;
    for (int64_t sl = lo; sl < hi; ++sl) {
        const float* x = a->x + sl * a->S;
        float* y = a->y ? a->y + sl * a->S : NULL;
        const int64_t c = sl % a->C;

        double sum = 0.0;
        for (int64_t i = 0; i < a->S; ++i) sum += (double)x[i];
        const double mean = sum / (double)a->S;

        double sq = 0.0;
        for (int64_t i = 0; i < a->S; ++i) {
            const double d = (double)x[i] - mean;
            sq += d * d;
        }
        const double var = sq / (double)a->S;
        const double inv = 1.0 / sqrt(var + a->eps);
        const double g = a->gamma ? (double)a->gamma[c] : 1.0;
        const double b = a->beta ? (double)a->beta[c] : 0.0;

        if (y)
            for (int64_t i = 0; i < a->S; ++i) y[i] = (float)(((double)x[i] - mean) * inv * g + b);
        if (a->mean_out) a->mean_out[sl] = mean;
        if (a->var_out) a->var_out[sl] = var;
    }
}

/* x, y: [slices, S] (slices = N*C, channel of a slice = slice % C). y may be NULL (stats only).
 * gamma/beta: [C] or NULL. mean_out/var_out: [slices] or NULL. Returns 0, or -1 on bad args. */
OR_API int or_instance_norm(const float* x, float* y, int64_t slices, int64_t C, int64_t S, double eps,
                            const float* gamma, const float* beta, double* mean_out, double* var_out,
                            int nthreads)
{
    if (!x || slices < 0 || C <= 0 || S <= 0) return -1;
    in_args a = {x, y, S, C, eps, gamma, beta, mean_out, var_out};
    parallel_for(slices, nthreads, in_range, &a);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Direct convolution, kernel 3, stride 1, no padding ("valid"), with bias.                   */
/*                                                                                            */
/* BN page, its direct-conv kernel discussion: out[n,k,oh,ow] = bias[k] + sum over input      */
/* channel c and taps (kh, kw) of W[k,c,kh,kw] * x[n,c,oh+kh,ow+kw] (cross-correlation, no    */
/* flip), weights laid out [C_out, C_in, 3, 3]. IN3d page, its shape walk-through: the 3-D    */
/* form adds a depth tap, output extent = input extent - 2 along each axis.                   */
/* The result is kept in fp64 (never rounded) for the normalization that follows.            */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    const float* x;
    const float* w;
    const float* b;
    double* out;
    int64_t N, Cin, Cout, D, H, W; /* D = 1 and dims = 2 for the 2-D form */
    int dims;
} conv_args;

static void conv_range(void* p, int64_t lo, int64_t hi)
{
    const conv_args* a = (const conv_args*)p;
    const int64_t KD = a->dims == 3 ? 3 : 1;
    const int64_t OD = a->D - KD + 1, OH = a->H - 2, OW = a->W - 2;
    for (int64_t nk = lo; nk < hi; ++nk) { /* one (n, k) output plane per step */
        const int64_t n = nk / a->Cout, k = nk % a->Cout;
        double* o = a->out + nk * OD * OH * OW;
        for (int64_t od = 0; od < OD; ++od)
            for (int64_t oh = 0; oh < OH; ++oh)
                for (int64_t ow = 0; ow < OW; ++ow) {
                    double acc = a->b ? (double)a->b[k] : 0.0;
                    for (int64_t c = 0; c < a->Cin; ++c)
                        for (int64_t kd = 0; kd < KD; ++kd)
                            for (int64_t kh = 0; kh < 3; ++kh)
                                for (int64_t kw = 0; kw < 3; ++kw) {
                                    const double wv =
                                        a->w[(((k * a->Cin + c) * KD + kd) * 3 + kh) * 3 + kw];
                                    const double xv =
                                        a->x[(((n * a->Cin + c) * a->D + od + kd) * a->H + oh + kh) *
                                                 a->W +
                                             ow + kw];
                                    acc += wv * xv;
                                }
                    o[(od * OH + oh) * OW + ow] = acc;
                }
    }
}

/* x: [N, Cin, (D,) H, W]; w: [Cout, Cin, (3,) 3, 3]; b: [Cout] or NULL;
 * out: [N, Cout, (D-2,) H-2, W-2] in fp64. dims is 2 (D ignored, treated as 1) or 3. */
OR_API int or_conv_k3(const float* x, const float* w, const float* b, double* out, int dims, int64_t N,
                      int64_t Cin, int64_t Cout, int64_t D, int64_t H, int64_t W, int nthreads)
{
    if (!x || !w || !out || (dims != 2 && dims != 3) || N < 0 || Cin <= 0 || Cout <= 0 || H < 3 ||
        W < 3 || (dims == 3 && D < 3))
        return -1;
    conv_args a = {x, w, b, out, N, Cin, Cout, dims == 3 ? D : 1, H, W, dims};
    parallel_for(N * Cout, nthreads, conv_range, &a);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Training-mode batch normalization over (N, spatial) per channel, then a scale.             */
/*                                                                                            */
/* BN page, opening analysis: in training mode the output uses the batch statistics, mean    */
/* and biased variance per channel over all (n, h, w); y = (x - mean)/sqrt(var + eps) *       */
/* gamma + beta, and the model then multiplies by scaling_factor (2.0). eps = 1e-5.           */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    const double* x;
    float* y;
    int64_t N, C, S;
    double eps;
    const float* gamma;
    const float* beta;
    double scale;
    double* mean_out;
    double* var_out;
} bn_args;

static void bn_range(void* p, int64_t lo, int64_t hi)
{
    const bn_args* a = (const bn_args*)p;
    const double cnt = (double)(a->N * a->S);
    for (int64_t c = lo; c < hi; ++c) {
        double sum = 0.0;
        for (int64_t n = 0; n < a->N; ++n) {
            const double* x = a->x + (n * a->C + c) * a->S;
            for (int64_t i = 0; i < a->S; ++i) sum += x[i];
        }
        const double mean = sum / cnt;
        double sq = 0.0;
        for (int64_t n = 0; n < a->N; ++n) {
            const double* x = a->x + (n * a->C + c) * a->S;
            for (int64_t i = 0; i < a->S; ++i) {
                const double d = x[i] - mean;
                sq += d * d;
            }
        }
        const double var = sq / cnt;
        const double inv = 1.0 / sqrt(var + a->eps);
        const double g = a->gamma ? (double)a->gamma[c] : 1.0;
        const double b = a->beta ? (double)a->beta[c] : 0.0;
        if (a->y)
            for (int64_t n = 0; n < a->N; ++n) {
                const double* x = a->x + (n * a->C + c) * a->S;
                float* y = a->y + (n * a->C + c) * a->S;
                for (int64_t i = 0; i < a->S; ++i) y[i] = (float)(((x[i] - mean) * inv * g + b) * a->scale);
            }
        if (a->mean_out) a->mean_out[c] = mean;
        if (a->var_out) a->var_out[c] = var;
    }
}

/* x: [N, C, S] in fp64; y: [N, C, S] fp32 or NULL; gamma/beta: [C] or NULL;
 * mean_out/var_out: [C] or NULL. */
OR_API int or_batch_norm_train(const double* x, float* y, int64_t N, int64_t C, int64_t S, double eps,
                               const float* gamma, const float* beta, double scale, double* mean_out,
                               double* var_out, int nthreads)
{
    if (!x || N <= 0 || C <= 0 || S <= 0) return -1;
    bn_args a = {x, y, N, C, S, eps, gamma, beta, scale, mean_out, var_out};
    parallel_for(C, nthreads, bn_range, &a);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Running statistics of training-mode batch norm.                                            */
/*                                                                                            */
/* BN page, opening analysis: a training-mode step also moves the running mean and variance  */
/* toward the batch statistics with momentum 0.1 -- running = (1 - m) * running + m * batch   */
/* -- and the running variance takes the unbiased batch variance (biased * n / (n - 1)).      */
/* mean/var: [C] batch statistics (var biased); count: values per channel (>= 2).            */
/* ------------------------------------------------------------------------------------------ */
OR_API int or_bn_running_update(const double* mean, const double* var, int64_t C, int64_t count,
                                double momentum, float* running_mean, float* running_var)
{
    if (!mean || !var || !running_mean || !running_var || C < 0 || count < 2) return -1;
    for (int64_t c = 0; c < C; ++c) {
        const double unbiased = var[c] * (double)count / (double)(count - 1);
        running_mean[c] = (float)((1.0 - momentum) * (double)running_mean[c] + momentum * mean[c]);
        running_var[c] = (float)((1.0 - momentum) * (double)running_var[c] + momentum * unbiased);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* The general conv -> normalize -> epilogue chain.                                           */
/*                                                                                            */
/* Step order (both pages' models are instances of it):                                       */
/*   c  = conv_k3(x) + bias                         (both pages)                              */
/*   s  = c * pre_mul[k]                            (IN3d page: first multiply by multiplier) */
/*   z  = (s - mean) / sqrt(var + eps)              (IN3d: per (n,k) over space;              */
/*                                                   BN page: per k over (n, space))          */
/*   z  = z * gamma[k] + beta[k]                    (BN page: affine batch norm)              */
/*   z  = z * out_scale                             (BN page: x scaling_factor)               */
/*   z  = min(max(z, lo), hi)                       (IN3d page: clamp, its min(max()) order)  */
/*   u  = z * post_mul[k]                           (IN3d page: second multiply)              */
/*   out = max over k of u  (if reduce_max_c), else out = u laid out like c                   */
/* Every step is in fp64; one rounding to fp32 at the store.                                  */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    double* s; /* [N, Cout, SP] pre-multiplied conv output, fp64 */
    int64_t N, Cout, SP;
    int batch; /* 1: statistics per channel over (N, SP); 0: per (n, k) over SP */
    double eps;
    double* mean; /* [N*Cout] (instance) or [Cout] (batch) */
    double* inv;
} chain_stats_args;

static void chain_stats_range(void* p, int64_t lo, int64_t hi)
{
    const chain_stats_args* a = (const chain_stats_args*)p;
    for (int64_t u = lo; u < hi; ++u) {
        /* batch: u is a channel, the reduction runs over every n; instance: u is (n, k) */
        const int64_t n0 = a->batch ? 0 : u / a->Cout;
        const int64_t n1 = a->batch ? a->N : n0 + 1;
        const int64_t k = a->batch ? u : u % a->Cout;
        const double cnt = (double)((n1 - n0) * a->SP);
        double sum = 0.0;
        for (int64_t n = n0; n < n1; ++n) {
            const double* s = a->s + (n * a->Cout + k) * a->SP;
            for (int64_t i = 0; i < a->SP; ++i) sum += s[i];
        }
        const double mean = sum / cnt;
        double sq = 0.0;
        for (int64_t n = n0; n < n1; ++n) {
            const double* s = a->s + (n * a->Cout + k) * a->SP;
            for (int64_t i = 0; i < a->SP; ++i) {
                const double d = s[i] - mean;
                sq += d * d;
            }
        }
        a->mean[u] = mean;
        a->inv[u] = 1.0 / sqrt(sq / cnt + a->eps);
    }
}

typedef struct {
    const double* s;
    float* out;
    int64_t N, Cout, SP;
    int batch;
    const double* mean;
    const double* inv;
    const float* gamma;
    const float* beta;
    double out_scale;
    int clamp;
    double lo, hi;
    const float* post_mul;
    int reduce_max_c;
} chain_epi_args;

static double chain_value(const chain_epi_args* a, int64_t n, int64_t k, int64_t i)
{
    const int64_t st = a->batch ? k : n * a->Cout + k;
    double z = (a->s[(n * a->Cout + k) * a->SP + i] - a->mean[st]) * a->inv[st];
    if (a->gamma) z *= (double)a->gamma[k];
    if (a->beta) z += (double)a->beta[k];
    z *= a->out_scale;
    if (a->clamp) z = fmin(fmax(z, a->lo), a->hi);
    if (a->post_mul) z *= (double)a->post_mul[k];
    return z;
}

static void chain_epi_range(void* p, int64_t lo, int64_t hi)
{
    const chain_epi_args* a = (const chain_epi_args*)p;
    for (int64_t n = lo; n < hi; ++n) {
        if (a->reduce_max_c) {
            for (int64_t i = 0; i < a->SP; ++i) {
                double m = -INFINITY;
                for (int64_t k = 0; k < a->Cout; ++k) {
                    const double v = chain_value(a, n, k, i);
                    if (v > m) m = v;
                }
                a->out[n * a->SP + i] = (float)m;
            }
        } else {
            for (int64_t k = 0; k < a->Cout; ++k)
                for (int64_t i = 0; i < a->SP; ++i)
                    a->out[(n * a->Cout + k) * a->SP + i] = (float)chain_value(a, n, k, i);
        }
    }
}

typedef struct {
    double* c;
    const float* pre_mul;
    int64_t Cout, SP, total_planes;
} premul_args;

static void premul_range(void* p, int64_t lo, int64_t hi)
{
    const premul_args* a = (const premul_args*)p;
    for (int64_t pl = lo; pl < hi; ++pl) {
        const double m = (double)a->pre_mul[pl % a->Cout];
        double* c = a->c + pl * a->SP;
        for (int64_t i = 0; i < a->SP; ++i) c[i] *= m;
    }
}

/* x: [N, Cin, (D,) H, W]; w: [Cout, Cin, (3,) 3, 3]; b: [Cout] or NULL.
 * batch = 1: training-mode batch statistics per channel; 0: instance statistics per (n, k).
 * pre_mul, gamma, beta, post_mul: [Cout] or NULL. out: [N, SP'] if reduce_max_c else
 * [N, Cout, SP'] where SP' = (D-2)(H-2)(W-2) (3-D) or (H-2)(W-2) (2-D).
 * mean_out / inv_out (optional): the statistics of s, [N*Cout] (instance) or [Cout] (batch). */
OR_API int or_conv_norm_epilogue(const float* x, const float* w, const float* b, float* out, int dims,
                                 int64_t N, int64_t Cin, int64_t Cout, int64_t D, int64_t H, int64_t W,
                                 int batch, double eps, const float* pre_mul, const float* gamma,
                                 const float* beta, double out_scale, int clamp, double lo, double hi,
                                 const float* post_mul, int reduce_max_c, double* mean_out,
                                 double* inv_out, int nthreads)
{
    if (!out || N <= 0) return -1;
    const int64_t SP = (dims == 3 ? (D - 2) : 1) * (H - 2) * (W - 2);
    const int64_t nstat = batch ? Cout : N * Cout;
    double* c = (double*)malloc(sizeof(double) * (size_t)(N * Cout * SP));
    double* mean = (double*)malloc(sizeof(double) * (size_t)nstat);
    double* inv = (double*)malloc(sizeof(double) * (size_t)nstat);
    int rc = -1;
    if (!c || !mean || !inv) goto done;
    if (or_conv_k3(x, w, b, c, dims, N, Cin, Cout, D, H, W, nthreads) != 0) goto done;
    if (pre_mul) {
        premul_args pa = {c, pre_mul, Cout, SP, N * Cout};
        parallel_for(N * Cout, nthreads, premul_range, &pa);
    }
    {
        chain_stats_args sa = {c, N, Cout, SP, batch, eps, mean, inv};
        parallel_for(nstat, nthreads, chain_stats_range, &sa);
    }
    {
        chain_epi_args ea = {c,    out,       N,     Cout, SP, batch,    mean,        inv,
                             gamma, beta, out_scale, clamp, lo,   hi, post_mul, reduce_max_c};
        parallel_for(N, nthreads, chain_epi_range, &ea);
    }
    if (mean_out) memcpy(mean_out, mean, sizeof(double) * (size_t)nstat);
    if (inv_out) memcpy(inv_out, inv, sizeof(double) * (size_t)nstat);
    rc = 0;
done:
    free(c);
    free(mean);
    free(inv);
    return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Conv followed by eval-mode batch norm (running statistics), then a scale.                 */
/*                                                                                            */
/* BN page, its eval-mode discussion: in eval mode the norm uses the running statistics,     */
/* y = ((conv(x) - running_mean) / sqrt(running_var + eps) * gamma + beta) * scale. The page */
/* folds this into the conv weights; the oracle keeps the unfolded definition (fp64 conv,    */
/* then the per-channel affine map, one final rounding).                                     */
/* ------------------------------------------------------------------------------------------ */
OR_API int or_conv_bn_eval(const float* x, const float* w, const float* b, const float* running_mean,
                           const float* running_var, const float* gamma, const float* beta,
                           double eps, double scale, float* out, int dims, int64_t N, int64_t Cin,
                           int64_t Cout, int64_t D, int64_t H, int64_t W, int nthreads)
{
    if (!out || !running_mean || !running_var || N <= 0) return -1;
    const int64_t SP = (dims == 3 ? (D - 2) : 1) * (H - 2) * (W - 2);
    double* c = (double*)malloc(sizeof(double) * (size_t)(N * Cout * SP));
    if (!c) return -1;
    if (or_conv_k3(x, w, b, c, dims, N, Cin, Cout, D, H, W, nthreads) != 0) {
        free(c);
        return -1;
    }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < Cout; ++k) {
            const double inv = 1.0 / sqrt((double)running_var[k] + eps);
            const double g = gamma ? (double)gamma[k] : 1.0;
            const double bt = beta ? (double)beta[k] : 0.0;
            const double* cp = c + (n * Cout + k) * SP;
            float* op = out + (n * Cout + k) * SP;
            for (int64_t i = 0; i < SP; ++i)
                op[i] = (float)((((cp[i] - (double)running_mean[k]) * inv) * g + bt) * scale);
        }
    free(c);
    return 0;
}
