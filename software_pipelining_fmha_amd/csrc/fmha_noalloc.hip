// fmha_bwd_noalloc: the attention backward pass for callers that cannot
// allocate device memory. Its workspace (D_i and -lse_i * log2(e) per query
// row) lives in a fixed device array instead of a caller buffer; the kernels
// are those of fmha_bwd. The contract is stated in include/fmha.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "fmha.h"

namespace fmha_host {
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
              float scale);
int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, void* dq, void* dk, void* dv, float* ws, int B, int H, int N, int d,
            int causal, float scale, void* stream);
}  // namespace fmha_host

// The workspace: 2 floats per query row, one copy per GPU the library runs
// on, held until the process ends. In host code this name is a host-side
// stand-in, not a device address: host code only ever uses the per-device
// address that hipGetSymbolAddress returns for it.
static __device__ __align__(256) float scratch[2 * FMHA_BWD_NOALLOC_MAX_ROWS];

namespace {

// Device address of `scratch` on the current device. It is looked up on the
// first call made with that device current and cached; null if the lookup
// fails.
float* scratch_address() {
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    addr[dev] = static_cast<float*>(ptr);
  }
  return addr[dev];
}

}  // namespace

extern "C" int fmha_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                int B, int H, int N, int d, int causal, float scale,
                                void* stream) {
  if (B < 0 || H < 0 || N < 0) return FMHA_ERR_INVALID_ARGUMENT;
  if (B == 0 || H == 0 || N == 0) return FMHA_OK;
  const int st = fmha_host::check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale);
  if (st != FMHA_OK) return st;
  if (static_cast<int64_t>(B) * H * N > FMHA_BWD_NOALLOC_MAX_ROWS) return FMHA_ERR_TOO_LARGE;
  // The first kernel of the pass writes every workspace value the later ones
  // read, so nothing carried over from an earlier call is ever read and
  // nothing needs clearing.
  float* ws = scratch_address();
  if (!ws) return FMHA_ERR_HIP;
  return fmha_host::run_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, d, causal, scale,
                            stream);
}
