/*
 * oracle_gemm.c -- CPU oracle for the tiled FP16 GEMM  C = epi(alpha (A . B)).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (the plain definition the tiled method reaches):
 *   C[i][j] = rne16( epi( alpha * sum_{k=0}^{K-1} a(A[i][k]) * a(B[k][j]) ) )
 * - A is M x K and B is K x N, both row-major IEEE binary16 bit patterns.
 *   ("TileLang：比 Triton 低一层的 tile 语言", section "第一个 kernel：GEMM":
 *   each output tile is the product of an A row-panel and a B column-panel.)
 * - a() decodes binary16 exactly; the sum runs sequentially in k, in fp64.
 *   The pages keep the accumulator in fp32 and convert to fp16 only in the
 *   final copy ("5分钟上手TileLang：GPU内核开发指南", section "避坑与调参");
 *   the oracle uses fp64, which is at least as accurate, and rounds once.
 * - alpha scales the fp32 result block before anything else touches it, as
 *   the pages' FlashAttention forward scales its score block Q . K^T
 *   ("TileLang：比 Triton 低一层的 tile 语言", section "FlashAttention：在线
 *   softmax 写成 tile 代码").  alpha = 1 is the plain product.  The caller
 *   passes alpha's exact value (the library takes it as a binary32); the
 *   product with the fp64 sum is taken in fp64.
 * - epi is the identity or the ReLU max(x, 0) of the quickstart's fused
 *   epilogue ("TileLang：让GPU编程像Python一样简单的高性能计算新范式",
 *   section "并行计算的优雅表达"), applied after the scale.
 * - rne16 rounds to the nearest binary16 value, ties to even (IEEE default).
 *
 * Every product of two binary16 values is exact in binary64 (at most 22
 * significant bits), so FMA contraction or its absence gives the same bits.
 * Plain C, no SIMD intrinsics, no -ffast-math.  Work is split by output
 * rows over POSIX threads; no element's sum is reordered.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- binary16 codec --------------------------------------------------- */

/* Exact value of a binary16 bit pattern: sign bit 15, biased exponent
 * bits 14..10, fraction bits 9..0.  Subnormal: f * 2^-24.
 * Normal: (1024 + f) * 2^(e - 25).  e == 31: inf or NaN. */
double oracle_f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round a binary64 value to the nearest binary16, ties to even.
 * With E = max(floor(log2|x|), -14) the representable values near |x| are
 * the multiples of q = 2^(E-10); n = rint(|x| / q) is the rounded count
 * (|x|/q is exact: scaling by a power of two).  Because binary16 is
 * monotone in its bit pattern, the pattern is (E + 14) * 1024 + n; this
 * covers subnormals (E = -14), a carry to the next binade (n = 2048) and
 * overflow (pattern >= 0x7c00 means infinity). */
uint16_t oracle_f16_encode(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return s;
    if (isinf(a))
        return (uint16_t)(s | 0x7c00);
    int e2;
    frexp(a, &e2);           /* a = fr * 2^e2, fr in [0.5, 1) */
    int E = e2 - 1;          /* floor(log2 a) */
    if (E < -14)
        E = -14;
    double n = nearbyint(ldexp(a, 10 - E));
    long bits = (long)(E + 14) * 1024 + (long)n;
    if (bits >= 0x7c00)
        return (uint16_t)(s | 0x7c00);
    return (uint16_t)(s | (uint16_t)bits);
}

void oracle_f16_decode_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_decode(h[i]);
}

void oracle_f16_encode_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_encode(x[i]);
}

/* ---- threads ------------------------------------------------------------ */

int oracle_cpu_threads(void)
{
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0)
            return c;
    }
    return 1;
}

/* ---- GEMM --------------------------------------------------------------- */

typedef struct {
    const uint16_t *A;      /* M x K */
    const double *Bsel;     /* K x ncols: decoded B restricted to the chosen columns */
    uint16_t *C;            /* nrows x ncols */
    const int64_t *rows;    /* which A rows, length nrows */
    int64_t K, ncols;
    double scale;
    int relu;
    int64_t r_begin, r_end; /* this worker's slice of the nrows output rows */
    int status;
} oracle_job;

static void *oracle_worker(void *p)
{
    oracle_job *j = (oracle_job *)p;
    double *acc = (double *)malloc((size_t)(j->ncols > 0 ? j->ncols : 1) * sizeof(double));
    if (!acc) {
        j->status = -1;
        return NULL;
    }
    for (int64_t r = j->r_begin; r < j->r_end; ++r) {
        const uint16_t *arow = j->A + j->rows[r] * j->K;
        for (int64_t c = 0; c < j->ncols; ++c)
            acc[c] = 0.0;
        /* each acc[c] receives its K terms in order k = 0, 1, ..., K-1 */
        for (int64_t k = 0; k < j->K; ++k) {
            double a = oracle_f16_decode(arow[k]);
            const double *brow = j->Bsel + k * j->ncols;
            for (int64_t c = 0; c < j->ncols; ++c)
                acc[c] += a * brow[c];
        }
        uint16_t *crow = j->C + r * j->ncols;
        for (int64_t c = 0; c < j->ncols; ++c) {
            double v = j->scale * acc[c];
            if (j->relu)
                v = v > 0.0 ? v : 0.0;
            crow[c] = oracle_f16_encode(v);
        }
    }
    free(acc);
    j->status = 0;
    return NULL;
}

/* C[r][c] = rne16(epi(scale * sum_k A[rows[r]][k] * B[k][cols[c]])) for
 * the given row and column index lists (the full product when they are
 * 0..M-1 and 0..N-1).  Returns 0 on success, -1 on bad arguments or
 * allocation failure. */
int oracle_gemm_f16_sampled_scaled(int64_t M, int64_t N, int64_t K,
                                   const uint16_t *A, const uint16_t *B,
                                   const int64_t *rows, int64_t nrows,
                                   const int64_t *cols, int64_t ncols,
                                   double scale, int relu, uint16_t *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || ncols < 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    for (int64_t c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return -1;
    if (nrows == 0 || ncols == 0)
        return 0;

    /* decode the chosen columns of B once: Bsel[k][c] = a(B[k][cols[c]]) */
    double *Bsel = (double *)malloc((size_t)(K > 0 ? K : 1) * (size_t)ncols * sizeof(double));
    if (!Bsel)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t c = 0; c < ncols; ++c)
            Bsel[k * ncols + c] = oracle_f16_decode(B[k * N + cols[c]]);

    if (nthreads <= 0)
        nthreads = oracle_cpu_threads();
    if (nthreads > nrows)
        nthreads = (int)nrows;
    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(Bsel);
        free(jobs);
        free(tids);
        return -1;
    }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].A = A;
        jobs[t].Bsel = Bsel;
        jobs[t].C = C;
        jobs[t].rows = rows;
        jobs[t].K = K;
        jobs[t].ncols = ncols;
        jobs[t].scale = scale;
        jobs[t].relu = relu;
        jobs[t].r_begin = nrows * t / nthreads;
        jobs[t].r_end = nrows * (t + 1) / nthreads;
        jobs[t].status = -1;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, oracle_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    oracle_worker(&jobs[0]);
    /* run inline whatever could not get a thread */
    for (int t = started + 1; t < nthreads; ++t)
        oracle_worker(&jobs[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status != 0)
            rc = -1;
    free(Bsel);
    free(jobs);
    free(tids);
    return rc;
}

/* The unscaled block (scale 1). */
int oracle_gemm_f16_sampled(int64_t M, int64_t N, int64_t K,
                            const uint16_t *A, const uint16_t *B,
                            const int64_t *rows, int64_t nrows,
                            const int64_t *cols, int64_t ncols,
                            int relu, uint16_t *C, int nthreads)
{
    return oracle_gemm_f16_sampled_scaled(M, N, K, A, B, rows, nrows, cols, ncols, 1.0, relu, C, nthreads);
}

/* The full product: every row and every column. */
int oracle_gemm_f16_scaled(int64_t M, int64_t N, int64_t K,
                           const uint16_t *A, const uint16_t *B, double scale, int relu,
                           uint16_t *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    int64_t *rows = (int64_t *)malloc((size_t)M * sizeof(int64_t));
    int64_t *cols = (int64_t *)malloc((size_t)N * sizeof(int64_t));
    if (!rows || !cols) {
        free(rows);
        free(cols);
        return -1;
    }
    for (int64_t i = 0; i < M; ++i)
        rows[i] = i;
    for (int64_t j = 0; j < N; ++j)
        cols[j] = j;
    int rc = oracle_gemm_f16_sampled_scaled(M, N, K, A, B, rows, M, cols, N, scale, relu, C, nthreads);
    free(rows);
    free(cols);
    return rc;
}

int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t *A, const uint16_t *B, int relu,
                    uint16_t *C, int nthreads)
{
    return oracle_gemm_f16_scaled(M, N, K, A, B, 1.0, relu, C, nthreads);
}
