/*
 * CPU oracle for the fused multi-head attention forward and backward passes.
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
 *
 * Backward pass. Twill (OSDI'26), sections 6.3 and 6.4, schedules the
 * attention backward kernel on Hopper and Blackwell but prints no formula.
 * The gradients here are those of the scalar L = sum_{i,c} dO[i][c] * o_i[c]
 * with respect to q, k and v, written straight from the forward definition
 * above (chain rule through the softmax):
 *
 *   P_ij  = exp(s_ij - lse_i)                  (the softmax weight, j in J_i)
 *   D_i   = sum_c dO[i][c] * o_i[c]
 *   dP_ij = sum_c dO[i][c] * v[j][c]
 *   dS_ij = P_ij * (dP_ij - D_i)
 *   dq_i  = scale * sum_{j in J_i} dS_ij * k_j
 *   dk_j  = scale * sum_{i : j in J_i} dS_ij * q_i
 *   dv_j  = sum_{i : j in J_i} P_ij * dO_i
 *
 * lse_i and o_i are recomputed here from q, k, v, never taken from a caller.
 *
 * FP8 inputs. Tawa (CGO'26), section V-D, also measures attention with FP8
 * operands; the pages name no format. Here q, k, v may arrive as OCP FP8
 * E4M3 bytes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent 0 is subnormal, S.1111.111 is NaN, there is no infinity) with one
 * float descale per tensor: the value of byte x of q is descale_q * e4m3(x).
 * The attention is then the same definition on those values.
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

/* ------------------------------------------------------------------------- */
/* Backward pass                                                              */
/* ------------------------------------------------------------------------- */

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    int64_t H, N, d;
    int causal;
    double scale;
} head_args_t;

/* Forward quantities of query row i of head `head` (element offset of the
 * head): lse_i, D_i = dO_i . o_i and, if w_out is not NULL,
 * w_i = sum_c |dO[i][c]| * sum_j P_ij |v[j][c]| (how strongly D_i reacts to
 * relative errors in the entries of o_i; a tolerance scale for callers).
 * s and od are scratch of N and 2 d doubles. */
static void row_stats(const head_args_t *a, int64_t head, int64_t i, double *s, double *od,
                      double *lse_out, double *D_out, double *w_out)
{
    const int64_t N = a->N, d = a->d;
    const uint16_t *qi = a->q + head + i * d;
    const uint16_t *doi = a->dout + head + i * d;
    const int64_t nvis = a->causal ? i + 1 : N;

    for (int64_t j = 0; j < nvis; ++j) {
        const uint16_t *kj = a->k + head + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += g_half[qi[c]] * g_half[kj[c]];
        s[j] = a->scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    double *av = od + d; /* sum_j e_j |v_jc| */
    for (int64_t c = 0; c < d; ++c)
        od[c] = av[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double e = exp(s[j] - m);
        const uint16_t *vj = a->v + head + j * d;
        l += e;
        for (int64_t c = 0; c < d; ++c) {
            od[c] += e * g_half[vj[c]];
            av[c] += e * fabs(g_half[vj[c]]);
        }
    }
    double D = 0.0, w = 0.0;
    for (int64_t c = 0; c < d; ++c) {
        D += g_half[doi[c]] * (od[c] / l);
        w += fabs(g_half[doi[c]]) * (av[c] / l);
    }
    *lse_out = m + log(l);
    *D_out = D;
    if (w_out)
        *w_out = w;
}

/* dq_i of one query row, from the definition. s is scratch of N doubles.
 * If rss is not NULL it receives, per element, sqrt(sum_j (scale dS_ij k_jc)^2):
 * the root-sum-square of the terms (a tolerance scale for callers). If dsens
 * is not NULL it receives |scale| * w_i * sum_j P_ij |k_jc|, the bound on how
 * dq_i moves per unit relative error in o_i through D_i. */
static void dq_row(const head_args_t *a, int64_t head, int64_t i, double *s, double *od,
                   double *dq, double *rss, double *dsens)
{
    const int64_t d = a->d;
    const int64_t nvis = a->causal ? i + 1 : a->N;
    const uint16_t *doi = a->dout + head + i * d;
    double lse, D, w;
    row_stats(a, head, i, s, od, &lse, &D, &w); /* also leaves s_ij in s */
    if (dsens)
        for (int64_t c = 0; c < d; ++c)
            dsens[c] = 0.0;
    for (int64_t c = 0; c < d; ++c)
        dq[c] = 0.0;
    if (rss)
        for (int64_t c = 0; c < d; ++c)
            rss[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const uint16_t *vj = a->v + head + j * d;
        const uint16_t *kj = a->k + head + j * d;
        const double P = exp(s[j] - lse);
        double dP = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dP += g_half[doi[c]] * g_half[vj[c]];
        const double dS = P * (dP - D);
        for (int64_t c = 0; c < d; ++c)
            dq[c] += dS * g_half[kj[c]];
        if (rss)
            for (int64_t c = 0; c < d; ++c)
                rss[c] += (dS * g_half[kj[c]]) * (dS * g_half[kj[c]]);
        if (dsens)
            for (int64_t c = 0; c < d; ++c)
                dsens[c] += P * fabs(g_half[kj[c]]);
    }
    for (int64_t c = 0; c < d; ++c)
        dq[c] *= a->scale;
    if (rss)
        for (int64_t c = 0; c < d; ++c)
            rss[c] = fabs(a->scale) * sqrt(rss[c]);
    if (dsens)
        for (int64_t c = 0; c < d; ++c)
            dsens[c] *= fabs(a->scale) * w;
}

/* dk_j and dv_j of one key row. lse, D and W hold the row statistics of
 * every query row of the head. If rk / rv are not NULL they receive the
 * root-sum-square of the terms of each element, as in dq_row; if dsk is not
 * NULL it receives |scale| * sqrt(sum_i (P_ij w_i q_ic)^2), the root-sum-square
 * of the per-query D sensitivities of dk_j. */
static void dkdv_row(const head_args_t *a, int64_t head, int64_t j, const double *lse,
                     const double *D, const double *W, double *dk, double *dv, double *rk,
                     double *rv, double *dsk)
{
    const int64_t N = a->N, d = a->d;
    const uint16_t *kj = a->k + head + j * d;
    const uint16_t *vj = a->v + head + j * d;
    for (int64_t c = 0; c < d; ++c)
        dk[c] = dv[c] = 0.0;
    if (rk)
        for (int64_t c = 0; c < d; ++c)
            rk[c] = rv[c] = 0.0;
    if (dsk)
        for (int64_t c = 0; c < d; ++c)
            dsk[c] = 0.0;
    for (int64_t i = a->causal ? j : 0; i < N; ++i) {
        const uint16_t *qi = a->q + head + i * d;
        const uint16_t *doi = a->dout + head + i * d;
        double dot = 0.0, dP = 0.0;
        for (int64_t c = 0; c < d; ++c) {
            dot += g_half[qi[c]] * g_half[kj[c]];
            dP += g_half[doi[c]] * g_half[vj[c]];
        }
        const double P = exp(a->scale * dot - lse[i]);
        const double dS = P * (dP - D[i]);
        for (int64_t c = 0; c < d; ++c) {
            dv[c] += P * g_half[doi[c]];
            dk[c] += dS * g_half[qi[c]];
        }
        if (rk)
            for (int64_t c = 0; c < d; ++c) {
                rv[c] += (P * g_half[doi[c]]) * (P * g_half[doi[c]]);
                rk[c] += (dS * g_half[qi[c]]) * (dS * g_half[qi[c]]);
            }
        if (dsk)
            for (int64_t c = 0; c < d; ++c)
                dsk[c] += (P * W[i] * g_half[qi[c]]) * (P * W[i] * g_half[qi[c]]);
    }
    for (int64_t c = 0; c < d; ++c)
        dk[c] *= a->scale;
    if (rk)
        for (int64_t c = 0; c < d; ++c) {
            rk[c] = fabs(a->scale) * sqrt(rk[c]);
            rv[c] = sqrt(rv[c]);
        }
    if (dsk)
        for (int64_t c = 0; c < d; ++c)
            dsk[c] = fabs(a->scale) * sqrt(dsk[c]);
}

typedef struct {
    const head_args_t *a;
    int kind;             /* 0: row stats of a head, 1: dq rows, 2: dk/dv rows */
    int64_t head;         /* kind 0 */
    double *lse, *D, *W;  /* kind 0 output, kind 2 input */
    const int64_t *rows;  /* kinds 1, 2: n x 3 triples */
    const int64_t *heads; /* kind 2: head offset per row */
    const double *lse_of, *D_of, *W_of; /* kind 2: cached stats of the heads */
    double *out0, *out1;
    double *rss0, *rss1; /* optional root-sum-square outputs, NULL to skip */
    double *ds0;         /* optional D-sensitivity output, NULL to skip */
    int64_t begin, end;
    int status;
} bjob_t;

static void *bwd_worker(void *arg)
{
    bjob_t *jb = (bjob_t *)arg;
    const head_args_t *a = jb->a;
    double *s = (double *)malloc(sizeof(double) * (size_t)a->N);
    double *od = (double *)malloc(sizeof(double) * (size_t)(2 * a->d));
    if (!s || !od) {
        jb->status = 3;
        free(s);
        free(od);
        return NULL;
    }
    for (int64_t r = jb->begin; r < jb->end; ++r) {
        if (jb->kind == 0) {
            row_stats(a, jb->head, r, s, od, &jb->lse[r], &jb->D[r], &jb->W[r]);
        } else if (jb->kind == 1) {
            const int64_t *t = jb->rows + 3 * r;
            const int64_t head = (t[0] * a->H + t[1]) * a->N * a->d;
            dq_row(a, head, t[2], s, od, jb->out0 + r * a->d, jb->rss0 ? jb->rss0 + r * a->d : NULL,
                   jb->ds0 ? jb->ds0 + r * a->d : NULL);
        } else {
            const int64_t *t = jb->rows + 3 * r;
            const int64_t head = (t[0] * a->H + t[1]) * a->N * a->d;
            const int64_t hs = (t[0] * a->H + t[1]);
            /* lse_of / D_of are indexed by the head's slot in the cache */
            const int64_t slot = jb->heads[hs];
            dkdv_row(a, head, t[2], jb->lse_of + slot * a->N, jb->D_of + slot * a->N,
                     jb->W_of + slot * a->N, jb->out0 + r * a->d, jb->out1 + r * a->d,
                     jb->rss0 ? jb->rss0 + r * a->d : NULL, jb->rss1 ? jb->rss1 + r * a->d : NULL,
                     jb->ds0 ? jb->ds0 + r * a->d : NULL);
        }
    }
    free(s);
    free(od);
    return NULL;
}

/* Runs `proto` over [0, n) split across `threads` workers. */
static int run_jobs(const bjob_t *proto, int64_t n, int threads)
{
    if (n == 0)
        return 0;
    if (threads > n)
        threads = (int)n;
    bjob_t *jobs = (bjob_t *)calloc((size_t)threads, sizeof(bjob_t));
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
        jobs[t] = *proto;
        jobs[t].begin = n * t / threads;
        jobs[t].end = n * (t + 1) / threads;
        if (threads > 1 && pthread_create(&tids[t], NULL, bwd_worker, &jobs[t]) == 0)
            started[t] = 1;
        else
            bwd_worker(&jobs[t]);
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

static int rows_in_range(const int64_t *rows, int64_t n, int64_t B, int64_t H, int64_t N)
{
    for (int64_t r = 0; r < n; ++r) {
        const int64_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= N)
            return 0;
    }
    return 1;
}

/*
 * Gradients of L = sum(dO * O) for selected rows.
 *   q, k, v, dout : binary16 bit patterns, [B, H, N, d] contiguous
 *   qrows, n_q    : (b, h, i) triples; dq receives n_q x d doubles
 *   krows, n_k    : (b, h, j) triples; dk and dv receive n_k x d doubles each
 *   rss_q, rss_k, rss_v : NULL, or like dq, dk, dv: per element the
 *                   root-sum-square of the terms summed into it (tolerance
 *                   scale for a comparison with rounded arithmetic)
 *   ds_q, ds_k    : NULL, or like dq and dk: the D sensitivities described
 *                   at dq_row and dkdv_row (dv does not depend on D)
 *   threads       : worker threads (>= 1)
 * dk/dv rows need lse_i and D_i of every query row of their head, so each
 * distinct head among krows costs one full forward pass over that head.
 * Returns 0 on success, 1 on a bad argument (nothing written), 3 if memory
 * or a thread could not be had.
 */
int oracle_fmha_bwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *dout, int64_t B, int64_t H, int64_t N, int64_t d,
                         int causal, double scale, const int64_t *qrows, int64_t n_q,
                         double *dq, const int64_t *krows, int64_t n_k, double *dk,
                         double *dv, double *rss_q, double *rss_k, double *rss_v,
                         double *ds_q, double *ds_k, int threads)
{
    if (!q || !k || !v || !dout || B <= 0 || H <= 0 || N <= 0 || d <= 0 || n_q < 0 ||
        n_k < 0 || threads < 1 || (n_q > 0 && (!qrows || !dq)) ||
        (n_k > 0 && (!krows || !dk || !dv)))
        return 1;
    if (!rows_in_range(qrows, n_q, B, H, N) || !rows_in_range(krows, n_k, B, H, N))
        return 1;
    pthread_once(&g_half_once, build_half_table);

    head_args_t a = {q, k, v, dout, H, N, d, causal, scale};
    bjob_t proto;
    memset(&proto, 0, sizeof(proto));
    proto.a = &a;

    if ((rss_k == NULL) != (rss_v == NULL))
        return 1;
    proto.kind = 1;
    proto.rows = qrows;
    proto.out0 = dq;
    proto.rss0 = rss_q;
    proto.ds0 = ds_q;
    int st = run_jobs(&proto, n_q, threads);
    if (st || n_k == 0)
        return st;

    /* row statistics of every head that a dk/dv row belongs to */
    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B * H));
    if (!slot)
        return 3;
    for (int64_t x = 0; x < B * H; ++x)
        slot[x] = -1;
    int64_t n_heads = 0;
    for (int64_t r = 0; r < n_k; ++r) {
        const int64_t hs = krows[3 * r] * H + krows[3 * r + 1];
        if (slot[hs] < 0)
            slot[hs] = n_heads++;
    }
    double *lse = (double *)malloc(sizeof(double) * (size_t)(n_heads * N));
    double *D = (double *)malloc(sizeof(double) * (size_t)(n_heads * N));
    double *W = (double *)malloc(sizeof(double) * (size_t)(n_heads * N));
    if (!lse || !D || !W) {
        free(slot);
        free(lse);
        free(D);
        free(W);
        return 3;
    }
    for (int64_t hs = 0; hs < B * H && st == 0; ++hs) {
        if (slot[hs] < 0)
            continue;
        bjob_t sp = proto;
        sp.kind = 0;
        sp.head = hs * N * d;
        sp.lse = lse + slot[hs] * N;
        sp.D = D + slot[hs] * N;
        sp.W = W + slot[hs] * N;
        st = run_jobs(&sp, N, threads);
    }
    if (st == 0) {
        bjob_t kp = proto;
        kp.kind = 2;
        kp.rows = krows;
        kp.heads = slot;
        kp.lse_of = lse;
        kp.D_of = D;
        kp.W_of = W;
        kp.out0 = dk;
        kp.out1 = dv;
        kp.rss0 = rss_k;
        kp.rss1 = rss_v;
        kp.ds0 = ds_k;
        st = run_jobs(&kp, n_k, threads);
    }
    free(slot);
    free(lse);
    free(D);
    free(W);
    return st;
}

/* ------------------------------------------------------------------------- */
/* FP8 (OCP E4M3) inputs                                                      */
/* ------------------------------------------------------------------------- */

/* OCP FP8 E4M3 -> binary64, exact. */
static double decode_e4m3(uint8_t x)
{
    const int sign = x >> 7;
    const int expo = (x >> 3) & 0xf;
    const int frac = x & 0x7;
    double v;
    if (expo == 0xf && frac == 0x7)
        v = NAN;
    else if (expo == 0)
        v = ldexp((double)frac, -9);                  /* 0.frac * 2^-6 */
    else
        v = ldexp((double)(frac | 0x8), expo - 10);   /* 1.frac * 2^(e-7) */
    return sign ? -v : v;
}

void oracle_e4m3_to_double(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = decode_e4m3(src[i]);
}

typedef struct {
    const uint8_t *q, *k, *v;
    double dq, dk, dv; /* descales */
    int64_t H, N, d;
    int causal;
    double scale;
    const int64_t *rows;
    double *o, *lse, *rss_o, *rss_l, *sc_o, *sc_l;
    int64_t begin, end;
    int status;
} f8job_t;

static double g_e4m3[256];
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;

static void build_e4m3_table(void)
{
    for (int i = 0; i < 256; ++i)
        g_e4m3[i] = decode_e4m3((uint8_t)i);
}

/* One query row of the attention on the decoded, descaled values (the same
 * definition as one_row). If rss_o / rss_l are not NULL they receive a
 * tolerance scale for a kernel that rounds each weight P_ij to E4M3
 * (relative error <= 2^-4, absolute <= 2^-10 of the largest weight below the
 * normal range): with e_j = max(2^-4 P_ij, 2^-10 P_max),
 *   rss_o[c] = sqrt(sum_j e_j^2 (v_jc - o_c)^2),  rss_l = sqrt(sum_j e_j^2);
 * and sc_o / sc_l a scale for errors in the scores proportional to
 * a_j = |scale| * sum_c |q_c k_jc| (the sum of the magnitudes of the products):
 *   sc_o[c] = sum_j P_ij a_j |v_jc - o_c|,  sc_l = sum_j P_ij a_j. */
static void one_row_fp8(const f8job_t *jb, int64_t r, double *s)
{
    const int64_t b = jb->rows[3 * r + 0];
    const int64_t h = jb->rows[3 * r + 1];
    const int64_t i = jb->rows[3 * r + 2];
    const int64_t N = jb->N, d = jb->d;
    const int64_t head = (b * jb->H + h) * N * d;
    const uint8_t *qi = jb->q + head + i * d;
    const uint8_t *kh = jb->k + head;
    const uint8_t *vh = jb->v + head;
    double *o = jb->o + r * d;
    const int64_t nvis = jb->causal ? i + 1 : N;

    for (int64_t j = 0; j < nvis; ++j) {
        const uint8_t *kj = kh + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += (jb->dq * g_e4m3[qi[c]]) * (jb->dk * g_e4m3[kj[c]]);
        s[j] = jb->scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c)
        o[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double e = exp(s[j] - m);
        const uint8_t *vj = vh + j * d;
        l += e;
        for (int64_t c = 0; c < d; ++c)
            o[c] += e * (jb->dv * g_e4m3[vj[c]]);
    }
    for (int64_t c = 0; c < d; ++c)
        o[c] /= l;
    jb->lse[r] = m + log(l);

    if (jb->rss_o) {
        double *ro = jb->rss_o + r * d;
        double rl = 0.0;
        const double pmax = 1.0 / l; /* the largest weight: exp(m - m) / l */
        for (int64_t c = 0; c < d; ++c)
            ro[c] = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
            const double P = exp(s[j] - m) / l;
            const double e = fmax(0.0625 * P, 0.0009765625 * pmax);
            const uint8_t *vj = vh + j * d;
            rl += e * e;
            for (int64_t c = 0; c < d; ++c) {
                const double t = e * (jb->dv * g_e4m3[vj[c]] - o[c]);
                ro[c] += t * t;
            }
        }
        for (int64_t c = 0; c < d; ++c)
            ro[c] = sqrt(ro[c]);
        jb->rss_l[r] = sqrt(rl);

        double *so = jb->sc_o + r * d;
        double sl = 0.0;
        for (int64_t c = 0; c < d; ++c)
            so[c] = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
            const double P = exp(s[j] - m) / l;
            const uint8_t *kj = kh + j * d;
            const uint8_t *vj = vh + j * d;
            double a = 0.0;
            for (int64_t c = 0; c < d; ++c)
                a += fabs((jb->dq * g_e4m3[qi[c]]) * (jb->dk * g_e4m3[kj[c]]));
            a *= fabs(jb->scale);
            sl += P * a;
            for (int64_t c = 0; c < d; ++c)
                so[c] += P * a * fabs(jb->dv * g_e4m3[vj[c]] - o[c]);
        }
        jb->sc_l[r] = sl;
    }
}

static void *fp8_worker(void *arg)
{
    f8job_t *jb = (f8job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)jb->N);
    if (!s) {
        jb->status = 3;
        return NULL;
    }
    for (int64_t r = jb->begin; r < jb->end; ++r)
        one_row_fp8(jb, r, s);
    free(s);
    return NULL;
}

/*
 * Attention rows for FP8 inputs.
 *   q, k, v         : OCP E4M3 bytes, [B, H, N, d] contiguous
 *   dq, dk, dv      : per-tensor descales (value = descale * e4m3(byte))
 *   rows, n_rows    : (b, h, i) triples
 *   o, lse          : n_rows x d and n_rows doubles (output)
 *   rss_o, rss_l,
 *   sc_o, sc_l      : all NULL, or like o, lse, o, lse: the tolerance scales
 *                     described at one_row_fp8
 * Returns 0 on success, 1 on a bad argument, 3 if memory or a thread could
 * not be had.
 */
int oracle_fmha_fp8_rows(const uint8_t *q, const uint8_t *k, const uint8_t *v, double dq,
                         double dk, double dv, int64_t B, int64_t H, int64_t N, int64_t d,
                         int causal, double scale, const int64_t *rows, int64_t n_rows,
                         double *o, double *lse, double *rss_o, double *rss_l, double *sc_o,
                         double *sc_l, int threads)
{
    const int scales = rss_o != NULL;
    if (!q || !k || !v || !rows || !o || !lse || B <= 0 || H <= 0 || N <= 0 || d <= 0 ||
        n_rows < 0 || threads < 1 || scales != (rss_l != NULL) || scales != (sc_o != NULL) ||
        scales != (sc_l != NULL))
        return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= N)
            return 1;
    }
    pthread_once(&g_e4m3_once, build_e4m3_table);
    if (n_rows == 0)
        return 0;
    if (threads > n_rows)
        threads = (int)n_rows;
    f8job_t *jobs = (f8job_t *)calloc((size_t)threads, sizeof(f8job_t));
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
        f8job_t *jb = &jobs[t];
        jb->q = q; jb->k = k; jb->v = v;
        jb->dq = dq; jb->dk = dk; jb->dv = dv;
        jb->H = H; jb->N = N; jb->d = d;
        jb->causal = causal; jb->scale = scale;
        jb->rows = rows; jb->o = o; jb->lse = lse; jb->rss_o = rss_o; jb->rss_l = rss_l;
        jb->sc_o = sc_o; jb->sc_l = sc_l;
        jb->begin = n_rows * t / threads;
        jb->end = n_rows * (t + 1) / threads;
        if (threads > 1 && pthread_create(&tids[t], NULL, fp8_worker, jb) == 0)
            started[t] = 1;
        else
            fp8_worker(jb);
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
