// Fused multi-head attention forward pass for gfx950 (MI355X, CDNA4).
//
// One workgroup owns one (batch, head, query tile). The query tile stays in
// VGPRs for the whole kernel. Key/value tiles stream from HBM through a
// double-buffered LDS ring. Each pages' stage maps onto gfx950 units:
// - T stage, S = Q K^T (Tawa, section III-D): fp16 MFMA, fp32 accumulate;
// - C stage, online softmax with rescale (PipeThreader's softmax and
//   rescale tasks): VALU, exp2 on the transcendental unit;
// - U stage, O += P V: fp16 MFMA.
//
// Data layout choices (all in registers of one 64-lane wave):
// * Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_f16. A lane of the accumulator then holds 16 keys of
//   one query column. So the row max and row sum are in-lane reductions
//   plus one swap between the two 32-lane halves.
// * Key rows are written to LDS under a permutation that swaps bits 2 and 3
//   of the row index within each 32-row block. With it, accumulator register
//   i of lane-half h holds key 16*(i/8) + 8*h + i%8. Eight consecutive
//   registers therefore cover 8 consecutive keys. After conversion to fp16
//   they are the B operand of O^T += V^T P^T, with no shuffle.
// * V is stored transposed in LDS ([d][key], keys contiguous). One 16-byte
//   LDS read then yields the matching A operand (8 keys of one d column).
// * O^T accumulates with one query per lane column. The per-row rescale
//   factor is therefore a per-lane scalar.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));

struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;
  int N;            // sequence length (queries = keys)
  int n_qt;         // query tiles per head
  int total_wg;     // B * H * n_qt
  float scale_log2; // scale * log2(e): scores go to the base-2 domain
};

template <int D>
struct Tile {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int QW = 32;                 // query rows per wave
  static constexpr int BM = WAVES * QW;         // query rows per workgroup
  static constexpr int BN = 64;                 // keys per pipeline stage
  static constexpr int KSTEPS = D / 16;         // MFMA k-steps of QK^T
  static constexpr int DBLK = D / 32;           // 32-row blocks of O^T
  static constexpr int PSTEPS = BN / 16;        // MFMA k-steps of PV
  // LDS rows padded by 16 bytes. With it, 8 (or 16) consecutive lanes
  // reading 16 B at the same column of consecutive rows hit distinct banks.
  static constexpr int K_STRIDE = D + 8;        // halfs per key row
  static constexpr int VT_STRIDE = BN + 8;      // halfs per d row of V^T
  static constexpr int K_TILE = BN * K_STRIDE;  // halfs
  static constexpr int V_TILE = D * VT_STRIDE;  // halfs
  static constexpr int STAGE = K_TILE + V_TILE; // halfs per ring slot
  // K tile loader: 16-byte chunks, CPR per key row.
  static constexpr int CPR = D / 8;
  static constexpr int K_ROWS_PER_PASS = THREADS / CPR;
  static constexpr int K_PASSES = BN / K_ROWS_PER_PASS;
  // V tile loader: each unit is 4 keys x 8 d, transposed on the way to LDS.
  static constexpr int V_UNITS = (BN / 4) * (D / 8);
  static_assert(V_UNITS <= THREADS, "one V unit per thread at most");
  static_assert(BN % K_ROWS_PER_PASS == 0, "K loader covers the tile");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0): loads past `bytes` return zeros, so ragged tails
  // need no branches. Word 3 = 0x00020000 is the gfx9-family raw-buffer format.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)0x00020000);
}

__device__ __forceinline__ intx4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Value of x in the partner lane (lane ^ 32) via v_permlane32_swap. After the
// swap the two results hold {x[l], x[l^32]} in some order, so callers combine
// them with a symmetric operation.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of a key inside the LDS K tile: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int key_slot(int key) {
  const int flip = ((key >> 2) ^ (key >> 3)) & 1;
  return key ^ (flip * 0xC);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fmha_fwd_kernel(Params p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work decomposition -------------------------------------------------
  // Workgroups go round-robin over the 8 XCDs (bid % 8). Renumber them so
  // that consecutive tile ids, i.e. the query tiles of one head, run on one
  // XCD and share its L2 copy of that head's K and V.
  const int G = p.total_wg;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int per = G >> 3, rem = G & 7;
  const int t = xcd * per + min(xcd, rem) + (bid >> 3);
  const int bh = t / p.n_qt;
  int qt = t - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // heaviest query tiles of a head first
  const int q0 = qt * T::BM;
  const int N = p.N;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + head, head_bytes);

  // ---- Q tile -> VGPRs: B operand of S^T = K Q^T ---------------------------
  // lane column = query (l32), lane half hh holds d = 16*s + 8*hh .. +7.
  const int qrow = q0 + wave * T::QW + l32;
  half8 qf[T::KSTEPS];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(half8, load16(rq, (qrow * D + 16 * s + 8 * hh) * 2));

  floatx16 oacc[T::DBLK];
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -INFINITY;  // running max of scaled scores (base-2 domain)
  float l_run = 0.f;        // this lane's share of the running sum

  const int n_kv_all = (N + T::BN - 1) / T::BN;
  const int n_kv = CAUSAL ? min(n_kv_all, (q0 + T::BM + T::BN - 1) / T::BN) : n_kv_all;

  // ---- K/V producer: HBM -> VGPRs -> LDS ring slot ---------------------------
  const int k_chunk = tid % T::CPR;
  const int k_row0 = tid / T::CPR;
  const int v_kg = tid % (T::BN / 4);  // keys 4*v_kg .. +3
  const int v_dg = tid / (T::BN / 4);  // d    8*v_dg .. +7
  const bool v_active = tid < T::V_UNITS;
  intx4 kreg[T::K_PASSES];
  intx4 vreg[4];

  auto fetch = [&](int j) {
    const int j0 = j * T::BN;
#pragma unroll
    for (int r = 0; r < T::K_PASSES; ++r)
      kreg[r] = load16(rk, ((j0 + k_row0 + r * T::K_ROWS_PER_PASS) * D + 8 * k_chunk) * 2);
    if (v_active) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = load16(rv, ((j0 + 4 * v_kg + r) * D + 8 * v_dg) * 2);
    }
  };
  auto stage = [&](int slot) {
    _Float16* ks = smem + slot * T::STAGE;
    _Float16* vt = ks + T::K_TILE;
#pragma unroll
    for (int r = 0; r < T::K_PASSES; ++r) {
      const int key = k_row0 + r * T::K_ROWS_PER_PASS;
      *reinterpret_cast<intx4*>(ks + key_slot(key) * T::K_STRIDE + 8 * k_chunk) = kreg[r];
    }
    if (v_active) {
      const half8 r0 = __builtin_bit_cast(half8, vreg[0]);
      const half8 r1 = __builtin_bit_cast(half8, vreg[1]);
      const half8 r2 = __builtin_bit_cast(half8, vreg[2]);
      const half8 r3 = __builtin_bit_cast(half8, vreg[3]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        half4 w = {r0[c], r1[c], r2[c], r3[c]};
        *reinterpret_cast<half4*>(vt + (8 * v_dg + c) * T::VT_STRIDE + 4 * v_kg) = w;
      }
    }
  };

  fetch(0);
  stage(0);
  if (n_kv > 1) fetch(1);
  __syncthreads();

  const float c2 = p.scale_log2;
  const int wave_q_lo = q0 + wave * T::QW;

  for (int j = 0; j < n_kv; ++j) {
    const _Float16* ks = smem + (j & 1) * T::STAGE;
    const _Float16* vt = ks + T::K_TILE;
    const int j0 = j * T::BN;

    // T stage: S^T = K Q^T for two 32-key blocks
    floatx16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < T::KSTEPS; ++s) {
        const half8 a = *reinterpret_cast<const half8*>(ks + (32 * kb + l32) * T::K_STRIDE + 16 * s + 8 * hh);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[s], sacc[kb], 0, 0, 0);
      }
    }

    // mask keys past N (ragged tail) and, if causal, keys after the query
    const bool need_mask = (j0 + T::BN > N) || (CAUSAL && j0 + T::BN - 1 > wave_q_lo);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
          if (key >= N || (CAUSAL && key > qrow)) sacc[kb][i] = -INFINITY;
        }
    }

    // C stage: online softmax in base 2
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
    half8 pf[T::PSTEPS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c2, -m_new));
        rs += e;
        pf[2 * kb + (i >> 3)][i & 7] = (_Float16)e;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b) oacc[b] *= alpha;

    // U stage: O^T += V^T P^T
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
      for (int s = 0; s < T::PSTEPS; ++s) {
        const half8 a = *reinterpret_cast<const half8*>(vt + (32 * b + l32) * T::VT_STRIDE + 16 * s + 8 * hh);
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[s], oacc[b], 0, 0, 0);
      }

    // producer: stage tile j+1 into the other slot, fetch tile j+2
    if (j + 1 < n_kv) {
      stage((j + 1) & 1);
      if (j + 2 < n_kv) fetch(j + 2);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, lse = (m + log2 l) * ln 2 -------------------
  const float l_tot = sum_halves(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    _Float16* orow = p.o + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        half4 w = {(_Float16)(oacc[b][4 * g + 0] * inv), (_Float16)(oacc[b][4 * g + 1] * inv),
                   (_Float16)(oacc[b][4 * g + 2] * inv), (_Float16)(oacc[b][4 * g + 3] * inv)};
        *reinterpret_cast<half4*>(orow + 32 * b + 8 * g + 4 * hh) = w;
      }
    if (hh == 0)
      p.lse[(size_t)bh * N + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

}  // namespace fmha
