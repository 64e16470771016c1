/*
 * CPU oracle for the fused multi-head attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench
 * script's CPU-baseline leg may load or call this file. The HIP library
 * never does, and this file includes nothing from it.
 *
 * What it computes. The pages split attention into three stages:
 * - Tawa (CGO'26), section III-D, coarse-grained pipeline: S = QK^T is the
 *   tensor-core stage T, softmax is the CUDA-core stage C, and the second
 *   product PV is the stage U;
 * - PipeThreader (OSDI'25), "core method": the tasks are load, mma,
 *   softmax and rescale.
 * The fused, tiled, online-softmax kernel reaches (up to rounding order) the
 * plain definition. So this oracle is that definition, in fp64, one query
 * row at a time. For query row i of head (b, h):
 *
 *   J     = {0..N-1}, or {0..i} when causal (key j visible iff j <= i)
 *   s_j   = scale * sum_c q[i][c] * k[j][c]          for j in J
 *   m     = max_j s_j,   e_j = exp(s_j - m),   l = sum_j e_j
 *   o[c]  = (sum_j e_j * v[j][c]) / l
 *   lse   = m + log(l)                               (natural log)
 *
 * Inputs are IEEE binary16 bit patterns in the [B, H, N, d] layout. They are
 * widened exactly to binary64. scale arrives as a double; callers pass the
 * float32 scale the kernel receives, widened.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE 754 binary16 -> binary64. Exact: every binary16 value is a binary64. */
static double decode_half(uint16_t h)
{
    const int sign = h >> 15;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* zero, subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac | 0x400), expo - 25); /* 1.frac * 2^(e-15) */
    return sign ? -v : v;
}

static double g_half[65536];
static pthread_once_t g_half_once = PTHREAD_ONCE_INIT;

static void build_half_table(void)
{
    for (uint32_t i = 0; i < 65536; ++i)
        g_half[i] = decode_half((uint16_t)i);
}

void oracle_half_to_double(const uint16_t *src, double *dst, int64_t n)
{
    pthread_once(&g_half_once, build_half_table);
    for (int64_t i = 0; i < n; ++i)
        dst[i] = g_half[src[i]];
}

typedef struct {
    const uint16_t *q, *k, *v;
    int64_t B, H, N, d;
    int causal;
    double scale;
    const int64_t *rows; /* n x 3: b, h, i */
    double *o;           /* n x d */
    double *lse;         /* n */
    int64_t begin, end;
    int status;
} job_t;

/* One query row, straight from the definition above. s and qd are scratch
 * of N and d doubles. */
static void one_row(const job_t *jb, int64_t r, double *s, double *qd)
{
    const int64_t b = jb->rows[3 * r + 0];
    const int64_t h = jb->rows[3 * r + 1];
    const int64_t i = jb->rows[3 * r + 2];
    const int64_t N = jb->N, d = jb->d;
    const int64_t head = (b * jb->H + h) * N * d;
    const uint16_t *qi = jb->q + head + i * d;
    const uint16_t *kh = jb->k + head;
    const uint16_t *vh = jb->v + head;
    double *o = jb->o + r * d;
    const int64_t nvis = jb->causal ? i + 1 : N;

    for (int64_t c = 0; c < d; ++c)
        qd[c] = g_half[qi[c]];

    /* scores */
    for (int64_t j = 0; j < nvis; ++j) {
        const uint16_t *kj = kh + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qd[c] * g_half[kj[c]];
        s[j] = jb->scale * dot;
    }

    /* softmax weights and the weighted sum of value rows */
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c)
        o[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double e = exp(s[j] - m);
        const uint16_t *vj = vh + j * d;
        l += e;
        for (int64_t c = 0; c < d; ++c)
            o[c] += e * g_half[vj[c]];
    }
    for (int64_t c = 0; c < d; ++c)
        o[c] /= l;
    jb->lse[r] = m + log(l);
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(jb->N > 0 ? jb->N : 1));
    double *qd = (double *)malloc(sizeof(double) * (size_t)jb->d);
    if (!s || !qd) {
        jb->status = 3;
        free(s);
        free(qd);
        return NULL;
    }
    for (int64_t r = jb->begin; r < jb->end; ++r)
        one_row(jb, r, s, qd);
    free(s);
    free(qd);
    return NULL;
}

/*
 * Computes n_rows query rows.
 *   q, k, v : binary16 bit patterns, [B, H, N, d] contiguous
 *   rows    : n_rows triples (b, h, i), each in range
 *   o       : n_rows x d doubles (output), lse: n_rows doubles (output)
 *   threads : worker threads (>= 1)
 * Returns 0 on success, 1 on a bad argument (nothing written), 3 if memory
 * or a thread could not be had.
 */
int oracle_fmha_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                     double scale, const int64_t *rows, int64_t n_rows,
                     double *o, double *lse, int threads)
{
    if (!q || !k || !v || !rows || !o || !lse || B <= 0 || H <= 0 || N <= 0 ||
        d <= 0 || n_rows < 0 || threads < 1)
        return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= N)
            return 1;
    }
    pthread_once(&g_half_once, build_half_table);
    if (n_rows == 0)
        return 0;
    if (threads > n_rows)
        threads = (int)n_rows;

    job_t *jobs = (job_t *)calloc((size_t)threads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    int *started = (int *)calloc((size_t)threads, sizeof(int));
    if (!jobs || !tids || !started) {
        free(jobs);
        free(tids);
        free(started);
        return 3;
    }
    int status = 0;
    for (int t = 0; t < threads; ++t) {
        job_t *jb = &jobs[t];
        jb->q = q; jb->k = k; jb->v = v;
        jb->B = B; jb->H = H; jb->N = N; jb->d = d;
        jb->causal = causal; jb->scale = scale;
        jb->rows = rows; jb->o = o; jb->lse = lse;
        jb->begin = n_rows * t / threads;
        jb->end = n_rows * (t + 1) / threads;
        if (threads == 1) {
            worker(jb);
        } else if (pthread_create(&tids[t], NULL, worker, jb) == 0) {
            started[t] = 1;
        } else {
            worker(jb); /* run it here rather than fail */
        }
    }
    for (int t = 0; t < threads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        if (jobs[t].status)
            status = jobs[t].status;
    }
    free(jobs);
    free(tids);
    free(started);
    return status;
}
