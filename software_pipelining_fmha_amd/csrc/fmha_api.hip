// C ABI of the attention forward and backward passes: argument checks,
// variant choice, and the launches on the caller's stream. The operations and
// the error contract are stated in include/fmha.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "fmha.h"
#include "fmha_bwd_kernel.hpp"
#include "fmha_fwd_fp8_kernel.hpp"
#include "fmha_fwd_kernel.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Compute units of the current device, rounded down to a multiple of 8 (one
// workgroup per CU for the persistent forward kernel; 8 XCDs). Cached per
// device; 0 if the query fails.
int persistent_grid() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int g = cus & ~7;
  if (dev >= 0 && dev < 64 && g > 0) cache[dev].store(g, std::memory_order_relaxed);
  return g;
}

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <int D, bool CAUSAL>
int launch(const fmha::Params& prm, hipStream_t stream) {
  using T = fmha::Tile<D>;
  void* args[] = {const_cast<fmha::Params*>(&prm)};
  // persistent: every tile if they fit in one wave of workgroups, else one
  // workgroup per CU (a multiple of 8), each walking several tiles
  const int cap = persistent_grid();
  if (cap <= 0) return FMHA_ERR_HIP;
  const int grid = prm.total_wg < cap ? prm.total_wg : cap;
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fmha::fmha_fwd_kernel<D, CAUSAL>),
                                       dim3(grid), dim3(T::THREADS), args, 0, stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

// Sign of a finite scale (-0 counts as 0) and the magnitude the forward
// kernels multiply by (1 for scale = 0, where Q is zeroed instead).
int scale_sign(float scale) { return scale > 0.f ? 1 : (scale < 0.f ? -1 : 0); }
double scale_magnitude(float scale) {
  return scale == 0.f ? 1.0 : std::fabs(static_cast<double>(scale));
}

}  // namespace

extern "C" int fmha_query_tile(int d) {
  if (d == 64) return fmha::Tile<64>::BM;
  if (d == 128) return fmha::Tile<128>::BM;
  return 0;
}

extern "C" int fmha_key_tile(int d) {
  if (d == 64) return fmha::Tile<64>::BN;
  if (d == 128) return fmha::Tile<128>::BN;
  return 0;
}

extern "C" int fmha_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, int causal, float scale, void* stream) {
  if (B < 0 || H < 0 || N < 0) return FMHA_ERR_INVALID_ARGUMENT;
  if (B == 0 || H == 0 || N == 0) return FMHA_OK;  // empty: nothing to do, pointers unused
  if (!q || !k || !v || !o || !lse) return FMHA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return FMHA_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return FMHA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FMHA_ERR_UNSUPPORTED;
  // byte offsets inside one head are 32-bit, with room for a ragged tile
  if ((static_cast<int64_t>(N) + 256) * d * 2 >= (int64_t(1) << 31)) return FMHA_ERR_UNSUPPORTED;

  const int bm = fmha_query_tile(d);
  const int64_t n_qt = (N + bm - 1) / bm;
  const int64_t grid = static_cast<int64_t>(B) * H * n_qt;
  if (grid >= (int64_t(1) << 31)) return FMHA_ERR_UNSUPPORTED;

  const uint64_t tbytes = static_cast<uint64_t>(B) * H * N * d * 2;
  const uint64_t lbytes = static_cast<uint64_t>(B) * H * N * 4;
  if (overlap(o, tbytes, q, tbytes) || overlap(o, tbytes, k, tbytes) || overlap(o, tbytes, v, tbytes) ||
      overlap(lse, lbytes, q, tbytes) || overlap(lse, lbytes, k, tbytes) ||
      overlap(lse, lbytes, v, tbytes) || overlap(lse, lbytes, o, tbytes))
    return FMHA_ERR_INVALID_ARGUMENT;

  fmha::Params prm;
  prm.q = static_cast<const _Float16*>(q);
  prm.k = static_cast<const _Float16*>(k);
  prm.v = static_cast<const _Float16*>(v);
  prm.o = static_cast<_Float16*>(o);
  prm.lse = lse;
  prm.N = N;
  prm.n_qt = static_cast<int>(n_qt);
  prm.total_wg = static_cast<int>(grid);
  // the kernel multiplies by |scale| and folds the sign into Q (scale = 0:
  // Q becomes 0 and any positive multiplier gives the same zero scores)
  prm.q_sign = scale_sign(scale);
  prm.scale_log2 = static_cast<float>(scale_magnitude(scale) * 1.4426950408889634);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 64) return causal ? launch<64, true>(prm, s) : launch<64, false>(prm, s);
  return causal ? launch<128, true>(prm, s) : launch<128, false>(prm, s);
}

namespace {

template <int D, bool CAUSAL>
int launch_bwd(const fmha::BwdParams& prm, hipStream_t stream) {
  using T = fmha::BwdTile<D>;
  void* args[] = {const_cast<fmha::BwdParams*>(&prm)};
  constexpr int rows_per_block = 256 / (D / 8);
  const int delta_grid = (prm.rows + rows_per_block - 1) / rows_per_block;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fmha::fmha_bwd_delta_kernel<D>),
                                 dim3(delta_grid), dim3(256), args, 0, stream);
  if (e != hipSuccess) return FMHA_ERR_HIP;
  static_assert(fmha::DkdvTile<D>::BT == T::BT, "both streaming kernels tile 128 rows");
  e = hipLaunchKernel(reinterpret_cast<const void*>(&fmha::fmha_bwd_dkdv_kernel<D, CAUSAL>),
                      dim3(prm.total_wg), dim3(fmha::DkdvTile<D>::THREADS), args, 0, stream);
  if (e != hipSuccess) return FMHA_ERR_HIP;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&fmha::fmha_bwd_dq_kernel<D, CAUSAL>),
                      dim3(prm.total_wg), dim3(fmha::DqTile<D>::THREADS), args, 0, stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

}  // namespace

extern "C" size_t fmha_bwd_workspace_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return static_cast<size_t>(2) * B * H * N * sizeof(float);
}

namespace fmha_host {

// Argument checks of the backward pass, shared by the entry points that take
// a workspace and that bring their own. ws is not examined here.
__attribute__((visibility("hidden"))) int check_bwd(const void* q, const void* k, const void* v,
                                                    const void* o, const void* dout,
                                                    const float* lse, void* dq, void* dk,
                                                    void* dv, int B, int H, int N, int d,
                                                    float scale) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FMHA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return FMHA_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return FMHA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return FMHA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(N) + 256) * d * 2 >= (int64_t(1) << 31)) return FMHA_ERR_UNSUPPORTED;
  const int64_t rows = static_cast<int64_t>(B) * H * N;
  if (rows >= (int64_t(1) << 30)) return FMHA_ERR_UNSUPPORTED;
  const int bt = fmha::BwdTile<128>::BT;
  const int64_t grid = static_cast<int64_t>(B) * H * ((N + bt - 1) / bt);
  if (grid >= (int64_t(1) << 31)) return FMHA_ERR_UNSUPPORTED;

  const uint64_t tb = static_cast<uint64_t>(rows) * d * 2;
  const uint64_t lb = static_cast<uint64_t>(rows) * 4;
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (void* out : outs) {
    for (const void* in : ins)
      if (overlap(out, tb, in, tb)) return FMHA_ERR_INVALID_ARGUMENT;
    if (overlap(out, tb, lse, lb)) return FMHA_ERR_INVALID_ARGUMENT;
    for (void* other : outs)
      if (other != out && overlap(out, tb, other, tb)) return FMHA_ERR_INVALID_ARGUMENT;
  }
  return FMHA_OK;
}

// The three launches, after the checks, with ws of 2 * B*H*N floats.
__attribute__((visibility("hidden"))) int run_bwd(const void* q, const void* k, const void* v,
                                                  const void* o, const void* dout,
                                                  const float* lse, void* dq, void* dk, void* dv,
                                                  float* ws, int B, int H, int N, int d,
                                                  int causal, float scale, void* stream) {
  const int64_t rows = static_cast<int64_t>(B) * H * N;
  const int bt = fmha::BwdTile<128>::BT;
  const int64_t n_t = (N + bt - 1) / bt;
  fmha::BwdParams prm;
  prm.q = static_cast<const _Float16*>(q);
  prm.k = static_cast<const _Float16*>(k);
  prm.v = static_cast<const _Float16*>(v);
  prm.o = static_cast<const _Float16*>(o);
  prm.dout = static_cast<const _Float16*>(dout);
  prm.lse = lse;
  prm.dq = static_cast<_Float16*>(dq);
  prm.dk = static_cast<_Float16*>(dk);
  prm.dv = static_cast<_Float16*>(dv);
  prm.ws = ws;
  prm.N = N;
  prm.rows = static_cast<int>(rows);
  prm.n_t = static_cast<int>(n_t);
  prm.total_wg = static_cast<int>(static_cast<int64_t>(B) * H * n_t);
  prm.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  prm.scale = scale;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 64) return causal ? launch_bwd<64, true>(prm, s) : launch_bwd<64, false>(prm, s);
  return causal ? launch_bwd<128, true>(prm, s) : launch_bwd<128, false>(prm, s);
}

}  // namespace fmha_host

using fmha_host::check_bwd;
using fmha_host::run_bwd;

extern "C" int fmha_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, float* ws, int B, int H,
                        int N, int d, int causal, float scale, void* stream) {
  if (B < 0 || H < 0 || N < 0) return FMHA_ERR_INVALID_ARGUMENT;
  if (B == 0 || H == 0 || N == 0) return FMHA_OK;
  if (!ws) return FMHA_ERR_INVALID_ARGUMENT;
  const int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale);
  if (st != FMHA_OK) return st;
  if (!aligned(ws, 4)) return FMHA_ERR_UNSUPPORTED;
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  const uint64_t tb = rows * d * 2, lb = rows * 4;
  const void* bufs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* b : bufs)
    if (overlap(ws, 2 * lb, b, tb)) return FMHA_ERR_INVALID_ARGUMENT;
  if (overlap(ws, 2 * lb, lse, lb)) return FMHA_ERR_INVALID_ARGUMENT;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, d, causal, scale, stream);
}

extern "C" int fmha_fwd_fp8(const void* q, const void* k, const void* v, float descale_q,
                            float descale_k, float descale_v, void* o, float* lse, int B, int H,
                            int N, int d, int causal, float scale, void* stream) {
  if (B < 0 || H < 0 || N < 0) return FMHA_ERR_INVALID_ARGUMENT;
  if (B == 0 || H == 0 || N == 0) return FMHA_OK;
  if (!q || !k || !v || !o || !lse) return FMHA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale) || !std::isfinite(descale_q) || !std::isfinite(descale_k) ||
      !std::isfinite(descale_v))
    return FMHA_ERR_INVALID_ARGUMENT;
  if (!(descale_q > 0.f) || !(descale_k > 0.f) || !(descale_v > 0.f)) return FMHA_ERR_UNSUPPORTED;
  if (d != fmha::Fp8Tile::D) return FMHA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FMHA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(N) + 256) * d * 2 >= (int64_t(1) << 31)) return FMHA_ERR_UNSUPPORTED;
  const int64_t n_qt = (N + fmha::Fp8Tile::BM - 1) / fmha::Fp8Tile::BM;
  const int64_t grid = static_cast<int64_t>(B) * H * n_qt;
  if (grid >= (int64_t(1) << 31)) return FMHA_ERR_UNSUPPORTED;
  const uint64_t ib = static_cast<uint64_t>(B) * H * N * d;  // fp8 input bytes
  const uint64_t ob = 2 * ib, lb = static_cast<uint64_t>(B) * H * N * 4;
  if (overlap(o, ob, q, ib) || overlap(o, ob, k, ib) || overlap(o, ob, v, ib) ||
      overlap(lse, lb, q, ib) || overlap(lse, lb, k, ib) || overlap(lse, lb, v, ib) ||
      overlap(lse, lb, o, ob))
    return FMHA_ERR_INVALID_ARGUMENT;

  fmha::Fp8Params prm;
  prm.q = static_cast<const uint8_t*>(q);
  prm.k = static_cast<const uint8_t*>(k);
  prm.v = static_cast<const uint8_t*>(v);
  prm.o = static_cast<_Float16*>(o);
  prm.lse = lse;
  prm.N = N;
  prm.n_qt = static_cast<int>(n_qt);
  prm.total_wg = static_cast<int>(grid);
  prm.scale_log2 = static_cast<float>(scale_magnitude(scale) * descale_q * descale_k *
                                      1.4426950408889634);
  prm.descale_v = descale_v;
  const int sign = scale_sign(scale);
  prm.q_and = sign == 0 ? 0u : 0xffffffffu;
  prm.q_xor = sign < 0 ? 0x80808080u : 0u;
  void* args[] = {&prm};
  const void* fn = causal ? reinterpret_cast<const void*>(&fmha::fmha_fwd_fp8_kernel<true>)
                          : reinterpret_cast<const void*>(&fmha::fmha_fwd_fp8_kernel<false>);
  const int cap = persistent_grid();
  if (cap <= 0) return FMHA_ERR_HIP;
  const int wgs = prm.total_wg < cap ? prm.total_wg : cap;
  const hipError_t e = hipLaunchKernel(fn, dim3(wgs), dim3(fmha::Fp8Tile::THREADS), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

extern "C" const char* fmha_status_str(int status) {
  switch (status) {
    case FMHA_OK: return "ok";
    case FMHA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FMHA_ERR_UNSUPPORTED: return "unsupported head dim, alignment, size or descale";
    case FMHA_ERR_HIP: return "HIP launch failed";
    case FMHA_ERR_TOO_LARGE: return "problem larger than the no-allocation entry point's workspace";
    default: return "unknown status";
  }
}
