/*
 * CPU oracle for the warp-specialised GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests and the bench script's
 * CPU-baseline leg may load or call this file. The HIP library never does,
 * and this file includes nothing from it.
 *
 * What it computes. The performance-model page for warp-specialised kernels
 * (section "GeMM and tiling") takes the general matrix product C = A x B
 * with A of M x K, B of K x N and C of M x N, tiled by (T_M, T_N, T_K). The
 * tiling only reorders the sums, so the oracle is the definition:
 *
 *   C[m][n] = sum_{k=0}^{K-1} A[m][k] * B[k][n]
 *
 * in fp64, one requested row m at a time, k in increasing order. It also
 * returns the magnitude sum
 *
 *   Cabs[m][n] = sum_k |A[m][k] * B[k][n]|
 *
 * which scales the rounding error any reordered fp32 sum may make. Inputs
 * are IEEE binary16 bit patterns, row-major (A[m][k] at m*K + k, B[k][n] at
 * k*N + n); they are widened exactly to binary64 (every binary16 value is a
 * binary64, and the product of two is exact in binary64).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* binary16 -> binary64, written out from the format: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 is subnormal, 31 is inf/NaN. */
static double gemm_half(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* every binary16 value, widened once */
static double g_gemm_half[65536];
static pthread_once_t g_gemm_once = PTHREAD_ONCE_INIT;

static void build_gemm_table(void)
{
    for (int h = 0; h < 65536; ++h)
        g_gemm_half[h] = gemm_half((uint16_t)h);
}

typedef struct {
    const uint16_t *a, *b;
    int64_t M, N, K;
    const int64_t *rows;
    int64_t n_rows;
    double *c, *cabs;
    int64_t first, last; /* this worker's share of the requested rows */
    int status;
} gemm_job_t;

static void *gemm_worker(void *arg)
{
    gemm_job_t *jb = (gemm_job_t *)arg;
    const int64_t N = jb->N, K = jb->K;
    /* Per requested row m: for k = 0, 1, ..., K-1 add A[m][k] * B[k][n] into
     * every column n. Each element's sum still runs over k in increasing
     * order; walking B row by row only keeps the reads contiguous. */
    for (int64_t r = jb->first; r < jb->last; ++r) {
        const int64_t m = jb->rows[r];
        double *c = jb->c + r * N, *ca = jb->cabs ? jb->cabs + r * N : NULL;
        for (int64_t n = 0; n < N; ++n) {
            c[n] = 0.0;
            if (ca)
                ca[n] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double am = g_gemm_half[jb->a[m * K + k]];
            const uint16_t *brow = jb->b + k * N;
            for (int64_t n = 0; n < N; ++n) {
                const double p = am * g_gemm_half[brow[n]];
                c[n] += p;
                if (ca)
                    ca[n] += fabs(p);
            }
        }
    }
    return NULL;
}

/*
 * oracle_gemm_rows: rows `rows[0..n_rows)` of C = A x B (and of Cabs, if
 * cabs is not NULL) into c[n_rows][N]. Returns 0, or -1 for an argument
 * error (a row outside [0, M), a negative size).
 */
int oracle_gemm_rows(const uint16_t *a, const uint16_t *b, int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t n_rows, double *c, double *cabs, int threads)
{
    if (M < 0 || N < 0 || K < 0 || n_rows < 0)
        return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    pthread_once(&g_gemm_once, build_gemm_table);
    if (threads < 1)
        threads = 1;
    if (threads > 64)
        threads = 64;
    if ((int64_t)threads > n_rows)
        threads = n_rows > 0 ? (int)n_rows : 1;
    gemm_job_t jobs[64];
    pthread_t tids[64];
    int started[64] = {0};
    for (int t = 0; t < threads; ++t) {
        jobs[t] = (gemm_job_t){a, b, M, N, K, rows, n_rows, c, cabs,
                               n_rows * t / threads, n_rows * (t + 1) / threads, 0};
        started[t] = pthread_create(&tids[t], NULL, gemm_worker, &jobs[t]) == 0;
        if (!started[t])
            gemm_worker(&jobs[t]);
    }
    int status = 0;
    for (int t = 0; t < threads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        if (jobs[t].status)
            status = jobs[t].status;
    }
    return status;
}
