/*
 * ws_gemm.h - C ABI of the warp-specialised GEMM for MI355X (gfx950) and of
 * the analytic performance model that picks its tile shape and ring depth.
 *
 * Source. The performance-model page for warp-specialised kernels (arXiv
 * 2506.11209, as summarised on the pages) describes:
 * - the kernel: C = A x B, tiled by (T_M, T_N, T_K); DMA warps load input
 *   tiles into a circular buffer in shared memory, MATH warps compute from
 *   it; wait/signal semaphores order them (sections "GeMM and tiling",
 *   "Warp specialization kernel structure", "Algorithm 1");
 * - the model: the wave count W, the stage count S, the linear timing
 *   primitives, the three coupled recurrences for the start times S_a, S_b,
 *   S_m, and a two-point calibration of throughputs (section "Core
 *   formulas").
 *
 * Status codes are those of fmha.h (0 ok, 1 invalid argument, 2
 * unsupported, 3 HIP launch failure).
 */
#ifndef WS_GEMM_H
#define WS_GEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ws_gemm - enqueue C = A x B on `stream`.
 *
 * a       : device pointer, binary16, row-major [M][K].
 * b       : device pointer, binary16, row-major [K][N].
 * c       : device pointer, binary16, row-major [M][N], written. Products
 *           accumulate in fp32 and are rounded to binary16 once.
 * M, N, K : sizes, each >= 0. If M or N is 0 nothing is enqueued and no
 *           pointer is examined. If K is 0, C is written with zeros and a, b
 *           are not examined. N and K must be multiples of 8 (16-byte rows);
 *           M is free.
 * tile_m, tile_n, tile_k, ring : the kernel variant, one of the list that
 *           ws_gemm_config returns (T_M in {64,128,256}, T_N in {64,128},
 *           T_K in {64,128}, ring depth 1..4 slots). All four 0 means: let
 *           ws_gemm_choose pick with the built-in MI355X model parameters.
 * trace   : NULL, or a device buffer of ws_gemm_trace_words(...) 64-bit
 *           words that receives per-stage timestamps (100 MHz wall clock):
 *           per workgroup, (S + 1) rows of 5 words. Row i < S: DMA wave
 *           0 starts issuing stage i; its share of stage i landed and
 *           signalled; MATH wave 0 starts stage i; MATH wave 0 releases its slot; MATH wave 0's
 *           MFMAs of stage i have finished (a traced launch waits for them
 *           each stage). Row S: the workgroup's start, its end, its tile
 *           id, 0, 0.
 * status  : NULL, or a device int the caller zeroes; set to 1 if a
 *           semaphore wait gave up (the output is then not valid). A wait
 *           gives up after about 2^22 polls, far beyond any legitimate wait.
 * stream  : hipStream_t (NULL = default stream).
 *
 * One workgroup (four DMA waves, four MATH waves) per output tile, at most
 * one per CU. The call allocates nothing, is asynchronous and thread-safe.
 * Buffers are caller-owned device memory; c must not overlap a or b.
 * Limits (else status 2): 16-byte aligned a, b, c; (M + 256) * K * 2 and
 * (K + 128) * N * 2 and M * N * 2 below 2^31 bytes.
 */
int ws_gemm(const void *a, const void *b, void *c, int M, int N, int K, int tile_m, int tile_n,
            int tile_k, int ring, unsigned long long *trace, int *status, void *stream);

/* ws_gemm_trace_words - 64-bit words of the trace buffer for a launch
 * (0 if the sizes or the variant are invalid). */
size_t ws_gemm_trace_words(int M, int N, int K, int tile_m, int tile_n, int tile_k);

/* ws_gemm_config_count / ws_gemm_config - the compiled kernel variants.
 * ws_gemm_config fills T_M, T_N, T_K and the ring depth of variant idx and
 * returns 0, or 1 if idx is out of range. */
int ws_gemm_config_count(void);
int ws_gemm_config(int idx, int *tile_m, int *tile_n, int *tile_k, int *ring);

/*
 * The analytic model (section "Core formulas"). Times are in microseconds,
 * sizes in matrix elements.
 *   T_MATH   = T_M T_N T_K / compute_throughput + compute_latency
 *   T_LOAD_A = T_M T_K / load_throughput + load_latency
 *   T_LOAD_B = T_K T_N / load_throughput + load_latency
 *   W = ceil(ceil(M / T_M) ceil(N / T_N) / n_units),  S = ceil(K / T_K)
 * with n_units the workgroups that run at once (one per CU here).
 */
typedef struct ws_model_params {
  double load_throughput;    /* elements per microsecond */
  double load_latency;       /* microseconds */
  double compute_throughput; /* multiply-adds per microsecond */
  double compute_latency;    /* microseconds */
  double t_epilogue;         /* microseconds per wave */
  double t_init;             /* microseconds per launch */
  int n_units;               /* concurrent workgroups */
} ws_model_params;

/*
 * ws_model_stage_times - the page's coupled recurrences for one workgroup
 * of S stages with a ring of `ring` slots (1-based i on the page, 0-based
 * arrays here):
 *   S_a(1) = 0
 *   S_a(i) = max(S_b(i-1) + T_LOAD_B, S_m(i-ring) + T_MATH)        (1)
 *   S_b(i) = max(S_a(i) + T_LOAD_A,   S_m(i-ring) + T_MATH)        (2)
 *   S_m(i) = max(S_m(i-1) + T_MATH,   S_b(i) + T_LOAD_B)           (3)
 * A term that refers to a stage before the first is absent (the page
 * leaves S_m(i - ring) for i <= ring undefined; no slot is then awaited).
 * s_a, s_b, s_m (each S doubles, or NULL) receive the start times. Returns
 * the end of the last MATH stage, S_m(S) + T_MATH (0 if S == 0), and the
 * total MATH wait in *math_wait (if not NULL): Wait(1) = S_b(1) + T_LOAD_B,
 * Wait(i) = S_m(i) - (S_m(i-1) + T_MATH). Returns -1 for S < 0 or ring < 1.
 */
double ws_model_stage_times(int S, int ring, double t_load_a, double t_load_b, double t_math,
                            double *s_a, double *s_b, double *s_m, double *math_wait);

/*
 * ws_model_launch_time - predicted time of one launch:
 *   (S_m(S) + T_MATH + T_EPILOGUE) W + T_INIT.
 * The page writes (S_m(S) + T_EPILOGUE) W + T_INIT; with S_m a start time
 * the last MATH stage's own duration is read into it. Returns -1 on
 * invalid arguments.
 */
double ws_model_launch_time(const ws_model_params *p, int M, int N, int K, int tile_m, int tile_n,
                            int tile_k, int ring);

/* ws_model_two_point - the page's two-point calibration of a linear
 * primitive time = size / throughput + latency from measurements
 * (size1, time1) and (size2, time2). Returns 0, or 1 if the two sizes or
 * times coincide. */
int ws_model_two_point(double size1, double time1, double size2, double time2,
                       double *throughput, double *latency);

/* ws_model_default - the built-in MI355X parameters (calibrated on the
 * device by the two-point method), for `cus` compute units. */
void ws_model_default(ws_model_params *p, int cus);

/* ws_gemm_choose - the compiled variant with the smallest predicted
 * launch time for (M, N, K) under *p (NULL = ws_model_default for the
 * current device); of equal predictions (relative 1e-9) for one tile shape,
 * the deepest ring. Returns 0, or an fmha.h status code. */
int ws_gemm_choose(const ws_model_params *p, int M, int N, int K, int *tile_m, int *tile_n,
                   int *tile_k, int *ring);

#ifdef __cplusplus
}
#endif

#endif /* WS_GEMM_H */
