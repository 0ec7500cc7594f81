/*
 * oracle_sparse.c -- CPU oracle for the 2:4 structured-sparse FP16 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle_gemm.c (whose binary16 codec it
 * uses): the slow, plain reference the GPU library is checked against.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * The pages name 2:4 sparse tensor-core GEMM (`T.gemm_sp`) as a TileLang
 * feature ("TileLang：让GPU编程像Python一样简单的高性能计算新范式", section
 * "高级特性超越基础矩阵乘法", sparse-compute paragraph) without fixing a
 * storage format.  This build reads it as follows:
 * - A (M x K) is 2:4 sparse along k: in every aligned group of 4 consecutive
 *   k at most 2 entries are kept.  K must be a multiple of 16.
 * - Compressed form: vals (M x K/2 binary16) holds, group after group, the 2
 *   kept values in increasing position order; meta (M x K/16 uint16) holds
 *   their positions: in word w of row i (dense k 16w .. 16w+15), bits
 *   2s+1..2s give the position (0..3) inside group 4w + s/2 of kept value s
 *   (s = 0..7) -- that is, value vals[i][8w + s] sits at
 *   k = 16w + 4 (s / 2) + pos.
 * - Compression keeps, in each group, the 2 entries of largest magnitude
 *   (ties: lower position first); a group with fewer nonzeros keeps zeros.
 *   Magnitudes are compared exactly, as binary16 bit patterns without the
 *   sign (monotone in |x| for non-NaN values).
 * - The product is the plain definition on the compressed operand:
 *     C[i][j] = rne16( epi( sum_w sum_s a(vals[i][8w+s]) * a(B[k(i,w,s)][j]) ) )
 *   summed in fp64 in order of w then s (increasing k when the two positions
 *   of a group differ), rounded once to nearest-even binary16.  For a
 *   compressed matrix this equals the dense oracle on its decompression.
 */
#define _GNU_SOURCE
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_decode(uint16_t h);
uint16_t oracle_f16_encode(double x);
int oracle_cpu_threads(void);

/* ---- compression ------------------------------------------------------- */

/* Positions (ascending) of the 2 kept entries of one group of 4. */
static void keep_two(const uint16_t *g, int *lo, int *hi)
{
    int first = 0;
    for (int p = 1; p < 4; ++p)
        if ((g[p] & 0x7fff) > (g[first] & 0x7fff))
            first = p;
    int second = first == 0 ? 1 : 0;
    for (int p = 0; p < 4; ++p)
        if (p != first && (g[p] & 0x7fff) > (g[second] & 0x7fff))
            second = p;
    *lo = first < second ? first : second;
    *hi = first < second ? second : first;
}

/* Compress a dense M x K binary16 matrix (K % 16 == 0): vals M x K/2,
 * meta M x K/16.  Returns 0, or -1 if K is not a multiple of 16. */
int oracle_sp_compress(int64_t M, int64_t K, const uint16_t *A, uint16_t *vals, uint16_t *meta)
{
    if (M < 0 || K < 0 || K % 16 != 0)
        return -1;
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t *row = A + i * K;
        for (int64_t w = 0; w < K / 16; ++w) {
            uint16_t word = 0;
            for (int q = 0; q < 4; ++q) {
                const uint16_t *g = row + 16 * w + 4 * q;
                int lo, hi;
                keep_two(g, &lo, &hi);
                vals[i * (K / 2) + 8 * w + 2 * q] = g[lo];
                vals[i * (K / 2) + 8 * w + 2 * q + 1] = g[hi];
                word |= (uint16_t)(lo << (4 * q));
                word |= (uint16_t)(hi << (4 * q + 2));
            }
            meta[i * (K / 16) + w] = word;
        }
    }
    return 0;
}

/* Dense M x K matrix holding each kept value at its position and +0
 * elsewhere.  Returns 0, or -1 if K % 16 != 0 or a group names one position
 * twice (such a group has no dense form with separate terms). */
int oracle_sp_decompress(int64_t M, int64_t K, const uint16_t *vals, const uint16_t *meta, uint16_t *A)
{
    if (M < 0 || K < 0 || K % 16 != 0)
        return -1;
    memset(A, 0, (size_t)(M * K) * sizeof(uint16_t));
    for (int64_t i = 0; i < M; ++i)
        for (int64_t w = 0; w < K / 16; ++w) {
            const uint16_t word = meta[i * (K / 16) + w];
            for (int q = 0; q < 4; ++q) {
                const int lo = (word >> (4 * q)) & 3, hi = (word >> (4 * q + 2)) & 3;
                if (lo == hi)
                    return -1;
                A[i * K + 16 * w + 4 * q + lo] = vals[i * (K / 2) + 8 * w + 2 * q];
                A[i * K + 16 * w + 4 * q + hi] = vals[i * (K / 2) + 8 * w + 2 * q + 1];
            }
        }
    return 0;
}

/* ---- product ------------------------------------------------------------ */

typedef struct {
    const uint16_t *vals, *meta;
    const double *Bsel;     /* K x ncols: decoded B restricted to the chosen columns */
    uint16_t *C;
    const int64_t *rows;
    int64_t K, ncols;
    int relu;
    int64_t r_begin, r_end;
    int status;
} sp_job;

static void *sp_worker(void *p)
{
    sp_job *j = (sp_job *)p;
    double *acc = (double *)malloc((size_t)(j->ncols > 0 ? j->ncols : 1) * sizeof(double));
    if (!acc) {
        j->status = -1;
        return NULL;
    }
    const int64_t W = j->K / 16;
    for (int64_t r = j->r_begin; r < j->r_end; ++r) {
        const uint16_t *vrow = j->vals + j->rows[r] * (j->K / 2);
        const uint16_t *mrow = j->meta + j->rows[r] * W;
        for (int64_t c = 0; c < j->ncols; ++c)
            acc[c] = 0.0;
        for (int64_t w = 0; w < W; ++w)
            for (int s = 0; s < 8; ++s) {
                const int pos = (mrow[w] >> (2 * s)) & 3;
                const int64_t k = 16 * w + 4 * (s / 2) + pos;
                const double a = oracle_f16_decode(vrow[8 * w + s]);
                const double *brow = j->Bsel + k * j->ncols;
                for (int64_t c = 0; c < j->ncols; ++c)
                    acc[c] += a * brow[c];
            }
        uint16_t *crow = j->C + r * j->ncols;
        for (int64_t c = 0; c < j->ncols; ++c) {
            double v = acc[c];
            if (j->relu)
                v = v > 0.0 ? v : 0.0;
            crow[c] = oracle_f16_encode(v);
        }
    }
    free(acc);
    j->status = 0;
    return NULL;
}

/* C[r][c] for the chosen rows and columns of the sparse product.  Returns 0,
 * or -1 on bad arguments (K % 16 != 0, index out of range) or allocation
 * failure. */
int oracle_gemm_f16_sp_sampled(int64_t M, int64_t N, int64_t K, const uint16_t *vals, const uint16_t *meta,
                               const uint16_t *B, const int64_t *rows, int64_t nrows, const int64_t *cols,
                               int64_t ncols, int relu, uint16_t *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || nrows < 0 || ncols < 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    for (int64_t c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return -1;
    if (nrows == 0 || ncols == 0)
        return 0;
    double *Bsel = (double *)malloc((size_t)(K > 0 ? K : 1) * (size_t)ncols * sizeof(double));
    if (!Bsel)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t c = 0; c < ncols; ++c)
            Bsel[k * ncols + c] = oracle_f16_decode(B[k * N + cols[c]]);
    int T = nthreads > 0 ? nthreads : oracle_cpu_threads();
    if (T > nrows)
        T = (int)nrows;
    sp_job *jobs = (sp_job *)calloc((size_t)T, sizeof(sp_job));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    if (!jobs || !th) {
        free(Bsel);
        free(jobs);
        free(th);
        return -1;
    }
    for (int t = 0; t < T; ++t)
        jobs[t] = (sp_job){vals, meta, Bsel, C, rows, K, ncols, relu, nrows * t / T, nrows * (t + 1) / T, -1};
    int started = 0;
    for (int t = 1; t < T; ++t) {
        if (pthread_create(&th[t], NULL, sp_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    sp_worker(&jobs[0]);
    /* run inline whatever could not get a thread */
    for (int t = started + 1; t < T; ++t)
        sp_worker(&jobs[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    int status = 0;
    for (int t = 0; t < T; ++t)
        if (jobs[t].status != 0)
            status = -1;
    free(Bsel);
    free(jobs);
    free(th);
    return status;
}

int oracle_gemm_f16_sp(int64_t M, int64_t N, int64_t K, const uint16_t *vals, const uint16_t *meta,
                       const uint16_t *B, int relu, uint16_t *C, int nthreads)
{
    if (M < 0 || N < 0)
        return -1;
    int64_t *rows = (int64_t *)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
    int64_t *cols = (int64_t *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int64_t));
    if (!rows || !cols) {
        free(rows);
        free(cols);
        return -1;
    }
    for (int64_t i = 0; i < M; ++i)
        rows[i] = i;
    for (int64_t j = 0; j < N; ++j)
        cols[j] = j;
    int st = oracle_gemm_f16_sp_sampled(M, N, K, vals, meta, B, rows, M, cols, N, relu, C, nthreads);
    free(rows);
    free(cols);
    return st;
}
