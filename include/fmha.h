/*
 * fmha.h - C ABI of the MI355X (gfx950) fused multi-head attention forward
 * and backward passes.
 *
 * The operation. For every batch b, head h and query row i:
 *   S   = scale * Q K^T      (one row: s_j = scale * q_i . k_j)
 *   P   = softmax(S)         (over the keys j visible to row i)
 *   O   = P V
 *   lse = log(sum_j exp(s_j))   (natural log of the scaled scores)
 * The pages split this into three stages. Tawa (CGO'26), section III-D,
 * coarse-grained pipeline: QK^T is the tensor-core stage T, softmax is the
 * stage C, and PV is the stage U. PipeThreader (OSDI'25) lists load, mma,
 * softmax and rescale tasks. Twill (OSDI'26), section 6.2, and Tawa,
 * section V-D, evaluate the FP16 forward kernel with batch 4, 32 heads and
 * head dim 128.
 *
 * The library computes it in one fused kernel. Each step of the path runs
 * in the library's own HIP kernels. It allocates no device memory at run
 * time and keeps no per-call state (fmha_bwd_noalloc's fixed workspace
 * aside).
 */
#ifndef FMHA_H
#define FMHA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by fmha_fwd. */
#define FMHA_OK 0
#define FMHA_ERR_INVALID_ARGUMENT 1 /* null pointer, negative size, non-finite scale, aliasing outputs */
#define FMHA_ERR_UNSUPPORTED 2      /* head dim, alignment, size or descale outside what the kernels handle */
#define FMHA_ERR_HIP 3              /* the kernel launch itself failed */

/*
 * fmha_fwd - enqueue the attention forward pass on `stream`.
 *
 * q, k, v : device pointers to IEEE binary16 tensors, contiguous [B, H, N, d]
 *           (row i of head (b, h) starts at ((b*H + h)*N + i)*d elements).
 *           Queries and keys have the same length N (self-attention).
 * o       : device pointer, binary16 [B, H, N, d], written.
 * lse     : device pointer, float32 [B, H, N], written. It holds the natural-log
 *           logsumexp of row i's scaled scores over its visible keys.
 * B, H, N : batch, heads, sequence length. Each must be >= 0. If any is 0 the
 *           call returns FMHA_OK and enqueues nothing; the pointers are then
 *           not examined (empty tensors may have null data pointers).
 * d       : head dimension, 64 or 128.
 * causal  : non-zero means key j is visible to query i only if j <= i (square,
 *           top-left aligned). Zero means every key is visible.
 * scale   : multiplier on q.k before the softmax; any finite value (the usual
 *           value is 1/sqrt(d); 0 gives uniform weights over the visible
 *           keys, a negative value favours the smallest q.k).
 * stream  : hipStream_t to enqueue on (NULL = the default stream).
 *
 * Ownership. All five buffers are caller-owned device memory on the current
 * device. Inputs are only read. o and lse must not overlap q, k, v or each
 * other. The call is asynchronous: it returns once the kernel is enqueued, and
 * outputs are valid after the stream is synchronised. It is thread-safe.
 *
 * Errors. On FMHA_ERR_INVALID_ARGUMENT or FMHA_ERR_UNSUPPORTED nothing is
 * enqueued and no HIP call is made. FMHA_ERR_HIP reports a failed launch.
 * Faults inside the kernel surface at the caller's next synchronisation.
 * Nothing is printed; no C++ exception crosses this boundary.
 *
 * Limits (else FMHA_ERR_UNSUPPORTED):
 * - q, k, v and o aligned to 16 bytes, lse to 4;
 * - (N + 256) * d * 2 < 2^31 bytes per head;
 * - the grid B*H*ceil(N/tile) < 2^31.
 */
int fmha_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int B, int H, int N, int d, int causal, float scale, void *stream);

/*
 * fmha_fwd_fp8 - the forward pass above with FP8 inputs (Tawa, CGO'26,
 * section V-D, measures FP8 attention; the pages name no format, so the OCP
 * FP8 E4M3 encoding with one descale per tensor is the reading taken).
 *
 * q, k, v    : device pointers to OCP E4M3 bytes, contiguous [B, H, N, d]. The
 *              value of byte x of q is descale_q * e4m3(x) (likewise k, v).
 * descale_*  : per-tensor descales, finite and > 0.
 * o, lse     : as for fmha_fwd (o binary16, lse float32 natural-log logsumexp
 *              of scale * q_i . k_j over the visible keys, descales included).
 * d          : 128 (the only head dim of this path).
 * Other arguments, ownership and errors as for fmha_fwd. Both products run on
 * the FP8 matrix core with fp32 accumulation; the softmax weights are rounded
 * to E4M3 before the second product, and the row sums add exactly those
 * rounded weights.
 */
int fmha_fwd_fp8(const void *q, const void *k, const void *v, float descale_q, float descale_k,
                 float descale_v, void *o, float *lse, int B, int H, int N, int d, int causal,
                 float scale, void *stream);

/*
 * fmha_bwd - enqueue the attention backward pass on `stream`.
 *
 * The gradients of the scalar sum_{b,h,i,c} dout[b,h,i,c] * o[b,h,i,c] with
 * respect to q, k and v, where o is the forward output above. Per head, with
 * P_ij = exp(scale * q_i . k_j - lse_i) over the visible keys:
 *   D_i  = dout_i . o_i
 *   dS_ij = P_ij * (dout_i . v_j - D_i)
 *   dq = scale * dS K,   dk = scale * dS^T Q,   dv = P^T dout.
 * Twill (OSDI'26), sections 6.3 and 6.4, schedules this backward kernel on
 * Hopper and Blackwell; the pages give no formula, so the one above is the
 * chain rule through the forward definition.
 *
 * q, k, v    : the forward inputs, binary16 [B, H, N, d] as for fmha_fwd.
 * o, lse     : the forward outputs for the same q, k, v, causal and scale
 *              (o binary16 [B, H, N, d], lse float32 [B, H, N]).
 * dout       : binary16 [B, H, N, d], the gradient of the loss with respect to o.
 * dq, dk, dv : binary16 [B, H, N, d], written.
 * ws         : float32 device workspace of fmha_bwd_workspace_bytes(B, H, N)
 *              bytes, caller-owned. The call overwrites it; on completion its
 *              first B*H*N values hold D_i = dout_i . o_i.
 * B, H, N, d, causal, scale, stream: as for fmha_fwd.
 *
 * Ownership and errors follow fmha_fwd: all buffers are caller-owned device
 * memory; dq, dk, dv and ws must not overlap the inputs or one another. It
 * launches three kernels in order on `stream` and allocates nothing. The
 * result is deterministic (no atomics). Limits as for fmha_fwd, and
 * B*H*N < 2^30.
 */
int fmha_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
             const float *lse, void *dq, void *dk, void *dv, float *ws,
             int B, int H, int N, int d, int causal, float scale, void *stream);

/* fmha_bwd_workspace_bytes - bytes of the ws argument of fmha_bwd
 * (2 * B * H * N floats; 0 if any size is <= 0). */
size_t fmha_bwd_workspace_bytes(int B, int H, int N);

/* fmha_status_str - static, human-readable text for a status code. */
const char *fmha_status_str(int status);

/* fmha_query_tile - query rows per workgroup of the kernel fmha_fwd launches
 * for head dim d (0 if d is unsupported). Bench and tests use it to size grids
 * and pick tile-edge rows. */
int fmha_query_tile(int d);

/* fmha_key_tile - keys per pipeline stage of that kernel (0 if unsupported). */
int fmha_key_tile(int d);

/* ---- no-allocation backward ----------------------------------------------
 * fmha_bwd_noalloc - fmha_bwd without the ws argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, and harnesses that forbid allocation.
 *
 * It runs the kernels of fmha_bwd on the same arguments (minus ws), with the
 * same results bit for bit, and makes no allocating call. Its workspace is a
 * fixed device array of 2 * FMHA_BWD_NOALLOC_MAX_ROWS floats (16 MiB), which
 * the library holds on every GPU it runs on until the process ends; the
 * first call on a device looks up its address there.
 *
 * Every call on one GPU shares that array: calls that overlap in time on one
 * GPU (on different streams, or from different threads onto unordered
 * streams) race and give wrong gradients. Calls ordered on one stream are
 * safe; each call rewrites every workspace value it reads.
 *
 * Errors as for fmha_bwd, plus FMHA_ERR_TOO_LARGE (nothing enqueued) when
 * B*H*N exceeds FMHA_BWD_NOALLOC_MAX_ROWS, and FMHA_ERR_HIP when the array's
 * address cannot be had on the current device.
 */
#define FMHA_ERR_TOO_LARGE 4 /* the problem exceeds a fixed internal buffer */
#define FMHA_BWD_NOALLOC_MAX_ROWS (1 << 21) /* B*H*N limit, e.g. B4 H32 N16384 */
int fmha_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                     const void *dout, const float *lse, void *dq, void *dk, void *dv,
                     int B, int H, int N, int d, int causal, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H */
