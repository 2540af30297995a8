/*
 * Plain CPU oracle for the fused quantized SwiGLU expansion.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library; the two meet only through
 * the seeded inputs.
 *
 * What it computes, in float64, one output element at a time:
 *
 *   code    q[n,k] = (W[n, k / (32/bits)] >> (bits * (k mod (32/bits)))) & (2^bits - 1)
 *   weight  w[n,k] = s[n, k/gs] * q[n,k] + b[n, k/gs]
 *   gate    g[m,n] = sum_k x[m,k] * wg[n,k]        (plain sequential sum)
 *   up      u[m,n] = sum_k x[m,k] * wu[n,k]
 *   MATCH   g~ = bf16_rne(g), u~ = bf16_rne(u);  others: g~ = g, u~ = u
 *   hidden  h[m,n] = g~ * sigma(g~) * u~,  sigma(t) = 1 / (1 + exp(-t))
 *
 * Sources (pages of the "mlx-bun" package diffs):
 *  - the operation and its unfused composition: "mlx-bun 0.0.7 -> 0.0.9"
 *    (page 43), qwen3.ts, the MLP forward (gate, up, sigmoid, two products);
 *    and the header comment of fused-swiglu-kernel.ts (page 42);
 *  - the packed layout: fused-swiglu-kernel.ts, host-entry docstring
 *    (weights [I, H*bits/32], scales and biases [I, H/groupSize]) and the
 *    per-row byte count of the kernel source;
 *  - affine zero-point "biases" added to scale*code: gemma4-base.ts,
 *    QuantizedLinear (page 42), and the support predicate requiring them;
 *  - the two precision variants (gate/up rounded to the activation dtype,
 *    or kept wide): fused-swiglu-kernel.ts, precision-variants comment;
 *  - bf16 or float16 activations, the kernel's element type being x's (so
 *    the scales, biases and result share it): fused-swiglu-kernel.ts,
 *    support predicate and the host entry's template dtype.
 * Readings where the pages are silent: codes least significant first in a
 * word; w = s*q + b with b added; bf16 and float16 rounding is
 * round-to-nearest-even.  "act" selects the activation type: 0 bf16, 1
 * IEEE binary16 (x, s and b read as that type; MATCH rounds to it).
 *
 * Also returned per element, for the comparison metric:
 *   nu_g[m,n] = sqrt(sum_k (x[m,k] * wg[n,k])^2), nu_u likewise.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- scalar helpers ---------------------------------------------------- */

/* bf16 bit pattern -> exact float64 value. */
double oracle_bf16_value(uint16_t bits)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)bits << 16;
    return (double)v.f;
}

/* float64 -> bf16, round to nearest, ties to even, directly from the double
 * (no intermediate float).  bf16 has an 8-bit significand and float's
 * exponent range: normal quantum 2^(e-7) for |v| in [2^e, 2^(e+1)),
 * subnormal quantum 2^-133.  Overflow gives +-inf; NaN stays NaN. */
uint16_t oracle_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7fc0;
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
    int qexp = (e - 1) - 7;           /* leading bit 2^(e-1), 7 more bits */
    if (qexp < -133)
        qexp = -133;
    double scaled = ldexp(a, -qexp);  /* exact: power-of-two scaling */
    double r = nearbyint(scaled);     /* default rounding mode: ties to even */
    double rounded = ldexp(r, qexp);
    if (rounded >= ldexp(1.0, 128))
        return sign | 0x7f80;         /* overflow to infinity */
    union { uint32_t u; float f; } out;
    out.f = (float)rounded;           /* exactly representable in float */
    return sign | (uint16_t)(out.u >> 16);
}

/* IEEE binary16 bit pattern -> exact float64 value: sign, 5-bit exponent
 * (bias 15), 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24),
 * exponent 31 infinity or NaN. */
double oracle_f16_value(uint16_t bits)
{
    double sign = (bits & 0x8000) ? -1.0 : 1.0;
    int e = (bits >> 10) & 0x1f;
    int f = bits & 0x3ff;
    if (e == 0)
        return sign * ldexp((double)f, -24);
    if (e == 31)
        return f ? NAN : sign * INFINITY;
    return sign * ldexp((double)(1024 + f), e - 25);
}

/* float64 -> binary16, round to nearest, ties to even, directly from the
 * double: normal quantum 2^(e-10) for |v| in [2^e, 2^(e+1)), subnormal
 * quantum 2^-24; a result of 2^16 or more (|v| >= 65520) is infinity. */
uint16_t oracle_f16_rne(double v)
{
    if (isnan(v))
        return 0x7e00;
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
    int qexp = (e - 1) - 10;          /* leading bit 2^(e-1), 10 more bits */
    if (qexp < -24)
        qexp = -24;
    double r = nearbyint(ldexp(a, -qexp));   /* ties to even */
    double rounded = ldexp(r, qexp);
    if (rounded >= 65536.0)
        return sign | 0x7c00;
    if (rounded < ldexp(1.0, -14))    /* subnormal (or rounded up to 2^-14: 0x0400) */
        return sign | (uint16_t)ldexp(rounded, 24);
    int ee;
    double mm = frexp(rounded, &ee);  /* rounded = mm * 2^ee */
    uint16_t frac = (uint16_t)ldexp(mm * 2.0 - 1.0, 10);
    return sign | (uint16_t)((ee - 1 + 15) << 10) | frac;
}

/* A 16-bit value of activation type act (0 bf16, 1 binary16), and the
 * rounding of a double to that type. */
static double act_value(uint16_t bits, int act)
{
    return act ? oracle_f16_value(bits) : oracle_bf16_value(bits);
}

static double act_round(double v, int act)
{
    return act ? oracle_f16_value(oracle_f16_rne(v)) : oracle_bf16_value(oracle_bf16_rne(v));
}

double oracle_sigmoid(double t) { return 1.0 / (1.0 + exp(-t)); }

double oracle_silu(double t) { return t * oracle_sigmoid(t); }

/* Code k of packed row n. */
uint32_t oracle_code(const uint32_t *W, int64_t H, int bits, int64_t n, int64_t k)
{
    int64_t per_word = 32 / bits;
    int64_t row_words = H / per_word;
    uint32_t word = W[n * row_words + k / per_word];
    return (word >> (bits * (int)(k % per_word))) & ((1u << bits) - 1u);
}

/* Dequantized weight w[n,k] = s * q + b (s and b of activation type act). */
static double weight_act(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                         int64_t H, int bits, int gs, int64_t n, int64_t k, int act)
{
    int64_t groups = H / gs;
    double s = act_value(S[n * groups + k / gs], act);
    double b = act_value(B[n * groups + k / gs], act);
    return s * (double)oracle_code(W, H, bits, n, k) + b;
}

double oracle_weight(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                     int64_t H, int bits, int gs, int64_t n, int64_t k)
{
    return weight_act(W, S, B, H, bits, gs, n, k, 0);
}

/* One quantized dot product: sum_k x[m,k] * w[n,k], and its scale nu. */
static void dot_one(const uint16_t *x, const uint32_t *W, const uint16_t *S,
                    const uint16_t *B, int64_t H, int bits, int gs,
                    int64_t m, int64_t n, int act, double *sum_out, double *nu_out)
{
    double sum = 0.0, sq = 0.0;
    for (int64_t k = 0; k < H; ++k) {
        double p = act_value(x[m * H + k], act) * weight_act(W, S, B, H, bits, gs, n, k, act);
        sum += p;
        sq += p * p;
    }
    *sum_out = sum;
    *nu_out = sqrt(sq);
}

/* ---- threaded drivers -------------------------------------------------- */

typedef struct {
    const uint16_t *x;
    const uint32_t *wg; const uint16_t *sg; const uint16_t *bg;
    const uint32_t *wu; const uint16_t *su; const uint16_t *bu;
    int64_t M, H, I;
    int bits_g, gs_g, bits_u, gs_u, mode, act;
    int64_t npairs;
    const int64_t *ms, *ns;       /* NULL: all pairs in row-major order */
    double *g, *u, *nu_g, *nu_u, *h;
    int64_t begin, end;
} job_t;

static void *pairs_worker(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t p = j->begin; p < j->end; ++p) {
        int64_t m = j->ms ? j->ms[p] : p / j->I;
        int64_t n = j->ns ? j->ns[p] : p % j->I;
        double g, u, nug, nuu;
        dot_one(j->x, j->wg, j->sg, j->bg, j->H, j->bits_g, j->gs_g, m, n, j->act, &g, &nug);
        dot_one(j->x, j->wu, j->su, j->bu, j->H, j->bits_u, j->gs_u, m, n, j->act, &u, &nuu);
        double gt = g, ut = u;
        if (j->mode == 0) {
            gt = act_round(g, j->act);
            ut = act_round(u, j->act);
        }
        if (j->g) j->g[p] = g;
        if (j->u) j->u[p] = u;
        if (j->nu_g) j->nu_g[p] = nug;
        if (j->nu_u) j->nu_u[p] = nuu;
        if (j->h) j->h[p] = oracle_silu(gt) * ut;
    }
    return NULL;
}

static int resolve_threads(int nthreads)
{
    if (nthreads > 0)
        return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int valid_spec(int64_t H, int bits, int gs)
{
    return (bits == 2 || bits == 4 || bits == 8) && gs > 0 && H > 0 && H % gs == 0 &&
           H % (32 / bits) == 0;
}

/*
 * Evaluate npairs output elements (ms[p], ns[p]); with ms == ns == NULL,
 * evaluate all M*I elements in row-major order (npairs must be M*I).
 * mode 0 = MATCH (gate/up rounded to the activation type), 1 and 2 = wide
 * gate/up; act 0 = bf16, 1 = binary16 activations, scales and biases.
 * Any of the output arrays may be NULL.  Returns 0, or -1 on bad arguments.
 */
int oracle_swiglu_pairs_act(const uint16_t *x,
                        const uint32_t *wg, const uint16_t *sg, const uint16_t *bg,
                        const uint32_t *wu, const uint16_t *su, const uint16_t *bu,
                        int64_t M, int64_t H, int64_t I,
                        int bits_g, int gs_g, int bits_u, int gs_u, int mode,
                        int64_t npairs, const int64_t *ms, const int64_t *ns,
                        double *g, double *u, double *nu_g, double *nu_u, double *h,
                        int act, int nthreads)
{
    if (!valid_spec(H, bits_g, gs_g) || !valid_spec(H, bits_u, gs_u))
        return -1;
    if (mode < 0 || mode > 2 || M < 0 || I < 0 || npairs < 0 || act < 0 || act > 1)
        return -1;
    if ((ms == NULL) != (ns == NULL))
        return -1;
    if (ms == NULL && npairs != M * I)
        return -1;
    for (int64_t p = 0; ms && p < npairs; ++p)
        if (ms[p] < 0 || ms[p] >= M || ns[p] < 0 || ns[p] >= I)
            return -1;
    if (npairs == 0)
        return 0;

    int nt = resolve_threads(nthreads);
    if (nt > npairs)
        nt = (int)npairs;
    job_t *jobs = (job_t *)calloc((size_t)nt, sizeof(job_t));
    pthread_t *tid = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    char *joined = (char *)calloc((size_t)nt, 1);
    if (!jobs || !tid || !joined) {
        free(jobs);
        free(tid);
        free(joined);
        return -1;
    }
    for (int t = 0; t < nt; ++t) {
        job_t *j = &jobs[t];
        j->x = x; j->wg = wg; j->sg = sg; j->bg = bg; j->wu = wu; j->su = su; j->bu = bu;
        j->M = M; j->H = H; j->I = I;
        j->bits_g = bits_g; j->gs_g = gs_g; j->bits_u = bits_u; j->gs_u = gs_u;
        j->mode = mode; j->act = act; j->npairs = npairs; j->ms = ms; j->ns = ns;
        j->g = g; j->u = u; j->nu_g = nu_g; j->nu_u = nu_u; j->h = h;
        j->begin = npairs * t / nt;
        j->end = npairs * (t + 1) / nt;
    }
    for (int t = 1; t < nt; ++t) {
        if (pthread_create(&tid[t], NULL, pairs_worker, &jobs[t]) == 0)
            joined[t] = 1;
        else
            pairs_worker(&jobs[t]);   /* no thread available: run inline */
    }
    pairs_worker(&jobs[0]);
    for (int t = 1; t < nt; ++t)
        if (joined[t])
            pthread_join(tid[t], NULL);
    free(joined);
    free(jobs);
    free(tid);
    return 0;
}

/* The bf16 form of oracle_swiglu_pairs_act. */
int oracle_swiglu_pairs(const uint16_t *x,
                        const uint32_t *wg, const uint16_t *sg, const uint16_t *bg,
                        const uint32_t *wu, const uint16_t *su, const uint16_t *bu,
                        int64_t M, int64_t H, int64_t I,
                        int bits_g, int gs_g, int bits_u, int gs_u, int mode,
                        int64_t npairs, const int64_t *ms, const int64_t *ns,
                        double *g, double *u, double *nu_g, double *nu_u, double *h,
                        int nthreads)
{
    return oracle_swiglu_pairs_act(x, wg, sg, bg, wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u, mode,
                                   npairs, ms, ns, g, u, nu_g, nu_u, h, 0, nthreads);
}

/*
 * Plain quantized matmul y[m,n] = sum_k x[m,k] * w[n,k] in float64, the single
 * projection the unfused composition applies twice (QuantizedLinear forward,
 * transposed weights).  Returns 0, or -1 on bad arguments.
 */
int oracle_qmm(const uint16_t *x, const uint32_t *W, const uint16_t *S, const uint16_t *B,
               int64_t M, int64_t H, int64_t N, int bits, int gs, double *y)
{
    if (!valid_spec(H, bits, gs) || M < 0 || N < 0)
        return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < H; ++k)
                s += oracle_bf16_value(x[m * H + k]) * oracle_weight(W, S, B, H, bits, gs, n, k);
            y[m * N + n] = s;
        }
    return 0;
}

/* Unpack every code of a [rows, H] packed matrix into bytes. */
int oracle_unpack(const uint32_t *W, int64_t rows, int64_t H, int bits, uint8_t *codes)
{
    if (!(bits == 2 || bits == 4 || bits == 8) || H % (32 / bits) != 0)
        return -1;
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t k = 0; k < H; ++k)
            codes[n * H + k] = (uint8_t)oracle_code(W, H, bits, n, k);
    return 0;
}

/* Vectorised helpers for the tests. */
void oracle_bf16_rne_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(v[i]);
}

void oracle_f16_rne_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_rne(v[i]);
}

void oracle_f16_value_array(const uint16_t *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_value(b[i]);
}

void oracle_silu_array(const double *v, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_silu(v[i]);
}
