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
// Register layouts (one 64-lane wave):
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

#include <type_traits>

namespace fmha {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// Reference-max slack (base 2) before O and l are rescaled.
constexpr float RESCALE_LOG2 = 8.0f;


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
  static constexpr int WAVES = 8;               // two groups of 4, one wave of each per SIMD
  static constexpr int THREADS = WAVES * 64;
  static constexpr int QW = 32;                 // query rows per wave
  static constexpr int BM = WAVES * QW;         // query rows per workgroup
  static constexpr int BN = 64;                 // keys per pipeline stage
  static constexpr int KB = BN / 32;            // 32-key MFMA blocks per stage
  static constexpr int KSTEPS = D / 16;         // MFMA k-steps of QK^T
  static constexpr int DBLK = D / 32;           // 32-row blocks of O^T
  static constexpr int PSTEPS = BN / 16;        // MFMA k-steps of PV
  static constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  static constexpr int TILE_BYTES = BN * D * 2; // one K tile in LDS
  static constexpr int VT_STRIDE = BN * 2 + 16; // bytes per d row of a V^T tile (16-byte pad)
  static constexpr int VT_BYTES = D * VT_STRIDE;  // one V^T tile in LDS
  static constexpr int SLOTS = 3;               // ring depth for K and for V^T
  static constexpr int LDS_BYTES = SLOTS * (TILE_BYTES + VT_BYTES);
  // V staging: each wave moves keys 8w .. 8w+7 of a tile; each lane 2 d columns
  static constexpr int V_KEYS_PER_WAVE = BN / WAVES;
  static constexpr int V_COLS = D / 64;          // d columns per lane (1 or 2)
  static_assert(V_KEYS_PER_WAVE == 8 && V_COLS * 64 == D, "V staging covers the tile");
  // one tile = TILE_BYTES / 1024 wave-wide 16-byte-per-lane LDS-DMA loads
  static constexpr int LOADS_PER_TILE = TILE_BYTES / 1024;
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TILE / WAVES;  // per tile
  static_assert(LOADS_PER_TILE % WAVES == 0 && LOADS_PER_WAVE >= 1, "tile loads split over waves");
  static_assert(LDS_BYTES <= 160 * 1024, "fits the CU's LDS");
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

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16*l (buffer_load_dwordx4 ... lds). lds_base must be uniform.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, int byte_off,
                                              __attribute__((address_space(3))) void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, byte_off, 0, 0, 0);
}

// Value of x combined with the partner lane (lane ^ 32) via v_permlane32_swap.
// After the swap the two results hold {x[l], x[l^32]} in some order, so they
// are combined with a symmetric operation.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key held by row p of an LDS K tile: bits 2 and 3 of p swapped (an involution).
__device__ __forceinline__ int key_of_row(int p) {
  const int flip = ((p >> 2) ^ (p >> 3)) & 1;
  return p ^ (flip * 0xC);
}

// LDS byte offset of 16-byte chunk c of row p in a K tile. The chunk index is
// XOR-swizzled with the row, so 16 lanes reading one chunk column of 16
// consecutive rows hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_chunk_off(int p, int c) {
  constexpr int CPR = D / 8;
  return (p * CPR + (c ^ (p % CPR))) * 16;
}

// LDS byte offset of 16-byte chunk c of key row `key` in a V tile (row-major,
// d contiguous). The swizzle 4*(key%4) makes the transposed 8-byte reads of
// 4 consecutive keys x 4 chunks (one ds_read_b64_tr_b16 half-wave) hit 16
// distinct bank groups.
template <int D>
__device__ __forceinline__ int v_chunk_off(int key, int c) {
  constexpr int CPR = D / 8;
  return (key * CPR + (c ^ ((4 * (key & 3)) % CPR))) * 16;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(Tile<D>::THREADS, 1) void fmha_fwd_kernel(Params p) {
  using T = Tile<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) half8 lds_half8;
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  // LDS: a 3-slot ring of K tiles and a 3-slot ring of V^T tiles.
  __shared__ __attribute__((aligned(16))) char smem_raw[T::LDS_BYTES];
  lds_char* const k_ring = (lds_char*)smem_raw;
  lds_char* const v_ring = k_ring + T::SLOTS * T::TILE_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;  // waves w and w + 4 share a SIMD
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
  const int wave_q_lo = q0 + wave * T::QW;
  const int qrow = wave_q_lo + l32;
  half8 qf[T::KSTEPS];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(half8, load16(rq, (qrow * D + 16 * s + 8 * hh) * 2));

  floatx16 oacc[T::DBLK];
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -INFINITY;  // reference max of scaled scores (base-2 domain)
  float l_run = 0.f;        // this lane's share of the running sum

  const int n_kv_all = (N + T::BN - 1) / T::BN;
  const int n_kv = CAUSAL ? min(n_kv_all, (q0 + T::BM + T::BN - 1) / T::BN) : n_kv_all;
  // Tiles this wave computes: causal rows see no key past wave_q_lo + 31.
  const int n_wave = CAUSAL ? min(n_kv, (wave_q_lo + T::QW - 1) / T::BN + 1) : n_kv;

  // ---- producers ---------------------------------------------------------------
  // K: HBM -> LDS ring slot by LDS-DMA, no register staging. Wave w issues
  // loads w*LOADS_PER_WAVE .. +LOADS_PER_WAVE-1 of a tile; load i fills the
  // tile's LDS chunks 64*i .. 64*i+63 (one per lane), and each lane fetches
  // the global chunk that the swizzled layout puts there.
  int k_src[T::LOADS_PER_WAVE];
#pragma unroll
  for (int r = 0; r < T::LOADS_PER_WAVE; ++r) {
    const int x = 64 * (wave * T::LOADS_PER_WAVE + r) + lane;  // LDS chunk index
    const int row = x / T::CPR, slot = x % T::CPR;
    k_src[r] = (key_of_row(row) * D + 8 * (slot ^ (row % T::CPR))) * 2;
  }
  auto fetch_k = [&](int j, int slot) __attribute__((always_inline)) {
    lds_char* dst = k_ring + slot * T::TILE_BYTES + wave * T::LOADS_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i)
      load16_to_lds(rk, j * T::BN * D * 2 + k_src[i], dst + i * 1024);
  };
  // V: HBM -> registers (keys 8w .. 8w+7 of the tile, d columns
  // V_COLS*lane .. +V_COLS-1), transposed in registers and written to a V^T
  // tile ([d][key], rows padded to VT_STRIDE bytes). The loads are coalesced
  // (a wave reads whole key rows); the A operand of PV is then one
  // ds_read_b128 of 8 consecutive keys of one d row.
  uint32_t vreg[T::V_KEYS_PER_WAVE];
  const int v_src = ((T::V_KEYS_PER_WAVE * wave) * D + T::V_COLS * lane) * 2;
  auto load_v = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < T::V_KEYS_PER_WAVE; ++r) {
      const int off = v_src + (j * T::BN + r) * D * 2;
      if constexpr (T::V_COLS == 2)
        vreg[r] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0);
      else
        vreg[r] = __builtin_amdgcn_raw_buffer_load_b16(rv, off, 0, 0);
    }
  };
  auto store_vt = [&](int slot) __attribute__((always_inline)) {
    lds_char* vt = v_ring + slot * T::VT_BYTES + (T::V_COLS * lane) * T::VT_STRIDE +
                   T::V_KEYS_PER_WAVE * wave * 2;
#pragma unroll
    for (int c = 0; c < T::V_COLS; ++c) {
      // key pairs (2i, 2i+1) of column c: half c of each loaded dword
      const uint32_t sel = c == 0 ? 0x05040100u : 0x07060302u;
      intx4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (int)__builtin_amdgcn_perm(vreg[2 * i + 1], vreg[2 * i], sel);
      *(__attribute__((address_space(3))) intx4*)(vt + c * T::VT_STRIDE) = w;
    }
  };

  // ---- consumer-side LDS offsets (per lane, constant over the loop) ----------
  // QK^T A operand: row 32*kb + l32 of the K tile, chunk 2*s + hh. The
  // swizzle depends on the row only through row % CPR, so the 32-row block kb
  // adds a constant.
  int k_rd[T::KSTEPS];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s) k_rd[s] = k_chunk_off<D>(l32, 2 * s + hh);
  constexpr int K_BLOCK_BYTES = 32 * T::CPR * 16;
  // PV A operand: V^T row 32*b + l32, keys 16*s + 8*hh .. +7 (16 bytes).
  const int vt_rd = l32 * T::VT_STRIDE + 16 * hh;

  floatx16 sacc[T::KB];   // S_j^T, then P_j in fp32
  half8 pf[T::PSTEPS];    // P_j^T in fp16: B operand of PV_j

  // T stage for key tile j: S^T = K_j Q^T.
  auto qk = [&](auto slot) __attribute__((always_inline)) {
    const lds_char* ks = k_ring + slot * T::TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const half8 a = *(const lds_half8*)(ks + k_rd[s] + kb * K_BLOCK_BYTES);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[s], sacc[kb], 0, 0, 0);
      }
  };
  // U stage for key tile j: O^T += V_j^T P_j^T.
  auto pv = [&](auto slot) __attribute__((always_inline)) {
    const lds_char* vs = v_ring + slot * T::VT_BYTES + vt_rd;
#pragma unroll
    for (int s = 0; s < T::PSTEPS; ++s)
#pragma unroll
      for (int b = 0; b < T::DBLK; ++b) {
        const half8 a = *(const lds_half8*)(vs + 32 * b * T::VT_STRIDE + 32 * s);
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[s], oacc[b], 0, 0, 0);
      }
  };

  const float c2 = p.scale_log2;
  const half2 ones = {(_Float16)1.f, (_Float16)1.f};

  // C stage, first half, for key tile j: mask, row max, lazy rescale and
  // p = 2^(s*c2 - m) in place (fp32).
  auto softmax_exp = [&](int j) __attribute__((always_inline)) {
    const int j0 = j * T::BN;
    // keys past N (ragged tail) and, if causal, keys after the query
    if ((j0 + T::BN > N) || (CAUSAL && j0 + T::BN - 1 > wave_q_lo)) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
          if (key >= N || (CAUSAL && key > qrow)) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    const float m_tile = max_halves(mx) * c2;
    // The reference max moves only when some row's max grows by more than
    // 2^RESCALE_LOG2. Until then p <= 2^RESCALE_LOG2; O and l share the same
    // reference, so O / l is unchanged and the rescale of O is skipped. O and l
    // already hold every earlier tile here (U_{j-1} ran before C_j).
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + RESCALE_LOG2) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < T::DBLK; ++b) oacc[b] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c2, -m_run));
  };
  // C stage, second half: P -> fp16 (the B operand of U) and its row sum.
  // The row sum adds the same fp16 weights that multiply V, in fp32.
  auto softmax_pack = [&]() __attribute__((always_inline)) {
    float rs[T::PSTEPS];
#pragma unroll
    for (int s = 0; s < T::PSTEPS; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[s][i] = (_Float16)sacc[s >> 1][8 * (s & 1) + i];
      rs[s] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2 pp = {pf[s][2 * e], pf[s][2 * e + 1]};
        rs[s] = __builtin_amdgcn_fdot2(pp, ones, rs[s], false);
      }
    }
    float rsum = rs[0];
#pragma unroll
    for (int s = 1; s < T::PSTEPS; ++s) rsum += rs[s];
    l_run += rsum;
  };

  // ---- ping-pong schedule -------------------------------------------------------
  // Every wave runs the same sequence of barrier-separated local intervals.
  // 2j is the matrix-core interval of iteration j: P_{j-1} -> fp16 and its row
  // sum (vector work that issues between the MFMAs), U_{j-1}, T_j. 2j+1 is the
  // vector interval: the producer work (write V^T_{j+1}, DMA K_{j+2}, load
  // V_{j+2}) and the first half of C_j (mask, max, lazy rescale, exp2).
  // Group 1 starts one interval late (an extra barrier up front, which group 0
  // matches at the end), so in every interval one wave of each SIMD feeds the
  // matrix core while the other runs the vector work.
  //
  // Rings (slot = tile % 3). K_j is read in global intervals 2j .. 2j+1 and
  // V^T_j in 2j+2 .. 2j+3. In local interval 2j+1 a wave writes V^T_{j+1}
  // (global 2j+1 or 2j+2) over V^T_{j-2}, last read in 2j-1, and DMAs K_{j+2}
  // over K_{j-1}, last read in 2j-1. A wave waits for its K_{j+1} DMA at the end
  // of local interval 2j and for its V^T writes at the end of each vector
  // interval; the barrier after each wait precedes the first read. Loads past
  // the sequence end return zeros into slots that are never read.
  auto sync = [&]() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
  auto mfma_sync = [&]() __attribute__((always_inline)) {
    // this wave's K_{j+1} DMA landed (its V_{j+1} register loads may not have)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(T::V_KEYS_PER_WAVE) : "memory");
  };
  auto vector_sync = [&]() __attribute__((always_inline)) {
    // this wave's V^T writes are in LDS
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto produce = [&](int j) __attribute__((always_inline)) {
    store_vt((j + 1) % T::SLOTS);
    fetch_k(j + 2, (j + 2) % T::SLOTS);
    load_v(j + 2);
  };

  // Steady-state iteration j (1 <= j < n_wave) with U = j % 3 known at
  // compile time, so every LDS operand address is a lane register plus an
  // immediate.
  auto steady = [&](int j, auto u_tag) __attribute__((always_inline)) {
    constexpr int U = decltype(u_tag)::value;
    constexpr int PREV = (U + 2) % 3;
    // local interval 2j: matrix core
    __builtin_amdgcn_s_setprio(1);
    softmax_pack();
    pv(std::integral_constant<int, PREV>{});
    qk(std::integral_constant<int, U>{});
    // Operand reads run 6 MFMAs ahead of their MFMA, with one vector
    // instruction of the P packing between consecutive MFMAs.
    constexpr int AHEAD = 6;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < T::PSTEPS * T::DBLK + T::KSTEPS * T::KB - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    mfma_sync();
    // local interval 2j+1: vector ALU
    produce(j);
    softmax_exp(j);
    vector_sync();
  };
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;

  fetch_k(0, 0);
  fetch_k(1, 1);
  load_v(0);
  store_vt(0);
  load_v(1);
  // K_0, K_1 landed and V^T_0 written (V_1 may still be in flight)
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(T::V_KEYS_PER_WAVE) : "memory");
  if (group == 1) sync();

  // j = 0: T_0, then C_0
  if (n_wave > 0) qk(U0{});
  mfma_sync();
  produce(0);
  if (n_wave > 0) softmax_exp(0);
  vector_sync();
  // 1 <= j < n_wave: P_{j-1}, U_{j-1}, T_j, then C_j
  int j = 1;
  for (; j + 3 <= n_wave; j += 3) {
    steady(j, U1{});
    steady(j + 1, U2{});
    steady(j + 2, U0{});
  }
  if (j < n_wave) {
    steady(j, U1{});
    ++j;
    if (j < n_wave) {
      steady(j, U2{});
      ++j;
    }
  }
  // n_wave <= j <= n_kv: the last U for this wave, then idle intervals in
  // which the wave still produces its share of the workgroup's tiles
  for (; j <= n_kv; ++j) {
    if (j == n_wave && j >= 1) {
      softmax_pack();
      pv((j - 1) % T::SLOTS);
    }
    mfma_sync();
    produce(j);
    vector_sync();
  }
  if (group == 0) sync();
  // no load may still be in flight when the workgroup exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
