// Fused multi-head attention forward pass with FP8 (OCP E4M3) Q, K and V, for
// gfx950 (MI355X, CDNA4). Head dim 128.
//
// Tawa (CGO'26), section V-D, measures this variant on Hopper. Here both
// products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, fp32
// accumulate, unit block scales), at twice the FP16 MFMA rate:
// - T stage, S^T = K Q^T: 2 key blocks x 2 k-steps of 64 bytes of d;
// - C stage: an exact pass (running max with lazy rescale, p <=
//   2^RESCALE_LOG2 = 256) and, as in the FP16 kernel, a fast pass whose
//   exponent reference stays at key tile 0's row max (no row max
//   afterwards). The weights are rounded to E4M3, whose conversion turns
//   values from 480 up into NaN (there is no infinity), so a fast-pass
//   overflow shows as a NaN row sum and the tile reruns exactly. The choice
//   is made per tile, from that tile's own data only;
// - U stage, O^T += V^T P^T: one MFMA per 32-row block of d per 64-key tile.
// Row sums of the E4M3 weights run on v_mfma_scale_f32_16x16x128_f8f6f4 with
// a 0/1 A operand, so O is normalised by exactly the weights that multiply V.
//
// Layouts. The MFMA pairs byte j of lane l in A with byte j of lane l in B;
// lanes l and l + 32 carry two disjoint halves of the 64 k values. So:
// - Q (B of S^T): lane l holds query l % 32, bytes d = 64 s + 32 (l / 32) ..
//   +31 of k-step s, straight from the Q row;
// - K (A of S^T): the same d bytes of key row key_of_row(l % 32) of the
//   32-key block, two ds_read_b128;
// - P^T (B of U): the fp32 score accumulator holds, in register i of
//   block kb, key 32 kb + 16 (i / 8) + 8 (l / 32) + i % 8 of query l % 32
//   (K rows are staged with bits 2 and 3 of the row swapped); byte
//   j = 16 kb + i of the packed weights is that key;
// - V^T (A of U): lane l needs d row l % 32 of the block and the same keys,
//   i.e. runs of 8 consecutive keys, which ds_read_b64_tr_b8 returns from V
//   in natural [key][d] layout: in each 16-lane group, source lane s reads 8
//   bytes of row s / 2, and result lane i receives byte i of each of the 8
//   rows.
// K and V tiles arrive by LDS-DMA into 4-slot rings with XOR-swizzled 16-byte
// chunks, so both kinds of read are free of bank conflicts.
#pragma once

#include "fmha_fwd_kernel.hpp"

namespace fmha {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx2 __attribute__((ext_vector_type(2)));

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  _Float16* o;
  float* lse;
  int N;             // sequence length
  int n_qt;          // query tiles per head
  int total_wg;      // B * H * n_qt
  float scale_log2;  // |scale| * descale_q * descale_k * log2(e) (> 0)
  float descale_v;
  // The sign of scale, folded into the Q bytes (E4M3 negation flips bit 7,
  // zero clears the byte; both exact): byte = (byte & q_and) ^ q_xor.
  uint32_t q_and;    // 0xffffffff, or 0 for scale = 0
  uint32_t q_xor;    // 0x80808080 for scale < 0, else 0
};

struct Fp8Tile {
  static constexpr int D = 128;
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int QW = 32;                   // query rows per wave
  static constexpr int BM = WAVES * QW;           // query rows per workgroup
  static constexpr int BN = 64;                   // keys per pipeline stage
  static constexpr int KB = BN / 32;              // 32-key blocks per stage
  static constexpr int KSTEPS = D / 64;           // 64-byte k-steps of QK^T
  static constexpr int DBLK = D / 32;             // 32-row blocks of O^T
  static constexpr int RUNS = BN / 16;            // runs of 8 keys per V^T operand half
  static constexpr int TILE_BYTES = BN * D;       // one K or V tile
  static constexpr int SLOTS = 4;                 // ring depth for K and for V
  static constexpr int RING_BYTES = SLOTS * TILE_BYTES;
  // O (fp16) is staged from the start of the V ring, rows padded by 16 bytes
  static constexpr int O_STRIDE = D * 2 + 16;
  static constexpr int O_STAGE_BYTES = WAVES * QW * O_STRIDE;
  static constexpr int LDS_BYTES = RING_BYTES + O_STAGE_BYTES;
  // K loads past the key sequence land in this 1 KB (inside the O staging,
  // past the V ring), not in the K ring that may hold the next tile's Q
  static constexpr int JUNK_OFFSET = 2 * RING_BYTES;
  static_assert(JUNK_OFFSET + 1024 <= LDS_BYTES, "junk line inside the LDS block");
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / WAVES;  // per tile
  static_assert(LOADS_PER_WAVE == 1, "one 16-byte DMA per lane per tile");
  // The next tile's Q: 4 KB per wave in the K ring, four 1 KB loads, load i
  // holding bytes 64 (i / 2) + 32 hh + 16 (i % 2) .. +15 of each lane's row
  static constexpr int Q_LOADS = QW * D / 1024;
  static_assert(WAVES * Q_LOADS * 1024 == RING_BYTES && Q_LOADS == 2 * KSTEPS, "one Q tile fills the K ring");
  // VMEM instructions of the epilogue, per wave: O rows and lse
  static constexpr int EPI_STORES = QW * D * 2 / 1024 + 1;
};

// 16-byte chunk swizzles (8 chunks per 128-byte row). K: 16 consecutive rows
// read at one chunk hit distinct banks. V: 8 consecutive rows read at two
// adjacent chunks (the transposing reads) hit distinct banks.
__device__ __forceinline__ int fp8_k_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int fp8_v_swz(int row) { return 2 * ((row >> 1) & 3); }

__device__ __forceinline__ floatx16 mfma_fp8(intx8 a, intx8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Pass choice. Every non-causal tile starts with the fast pass and reruns
// with the exact one when a weight overflowed, so a tile's output bits
// depend only on its own inputs (not on which tiles its workgroup ran
// before). E4M3's range is small (weights overflow past about 2^8.9 of the
// reference), so on sharp softmax rows most tiles pay for both passes. The
// causal kernel holds the exact pass only: with both passes compiled in, its
// exact pass ran 5% slower on sharp inputs.
// Non-causal tiles stage the next tile's Q rows in the idle K ring after
// their last T stage (t_next: -1 for none), and with q_staged a tile takes
// its Q from there, as the FP16 kernel does; the causal kernel loads Q at the
// tile's start.
template <bool CAUSAL>
__device__ __forceinline__ void fwd_fp8_tile(const Fp8Params& p, int t, int t_next, bool q_staged,
                                             char* smem_raw) {
  using T = Fp8Tile;
  constexpr int D = T::D;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) intx4 lds_intx4;
  typedef __attribute__((address_space(3))) intx2 lds_intx2;
  lds_char* const k_ring = (lds_char*)smem_raw;
  lds_char* const v_ring = k_ring + T::SLOTS * T::TILE_BYTES;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Non-causal: the lane index is formed per tile by an asm mbcnt the
  // compiler cannot hoist out of the tile loop (it would spill the hoisted
  // lane constants, as in the FP16 kernel).
  int lane;
  if constexpr (CAUSAL)
    lane = threadIdx.x & 63;
  else
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int group = wave >> 2;  // waves w and w + 4 share a SIMD
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bh = t / p.n_qt;
  int qt = t - bh * p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;
  const int q0 = qt * T::BM;
  const int N = p.N;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + head, head_bytes);

  // ---- Q tile -> VGPRs: B operand of S^T = K Q^T ---------------------------
  const int wave_q_lo = q0 + wave * T::QW;
  const int qrow = wave_q_lo + l32;
  intx8 qf[T::KSTEPS];
  constexpr bool STAGE_Q = !CAUSAL;
  static_assert(T::KSTEPS == 2, "four staged 16-byte reads");
  if (STAGE_Q && q_staged) {
    // the previous tile's epilogue (EPI_STORES stores) is all that was
    // issued since the staged loads; a barrier keeps the K ring from being
    // refilled before every wave has read its rows
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(T::EPI_STORES) : "memory");
    const uint32_t qs = (uint32_t)(uintptr_t)k_ring + wave * T::Q_LOADS * 1024 + 16 * lane;
    intx4 a0, a1, a2, a3;
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(qs)
        : "memory");
    asm volatile("s_barrier" ::: "memory");
    qf[0] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    qf[1] = __builtin_shufflevector(a2, a3, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s) {
      const intx4 a = load16(rq, qrow * D + 64 * s + 32 * hh);
      const intx4 b = load16(rq, qrow * D + 64 * s + 32 * hh + 16);
      qf[s] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  // The C stage needs a positive multiplier, so the sign of scale rides on Q.
  if (p.q_and != 0xffffffffu || p.q_xor != 0u) {
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (int)(((uint32_t)qf[s][e] & p.q_and) ^ p.q_xor);
  }

  floatx16 oacc[T::DBLK];
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -INFINITY;
  // Row sums of the E4M3 weights: v_mfma_scale_f32_16x16x128_f8f6f4 with P^T
  // (laid out for the 32x32x64 U MFMA) as B and E4M3 ones as A in lanes 0,
  // 32 (queries 0..15) and 20, 52 (queries 16..31): register 0 of lane q < 32
  // then holds query q's sum.
  floatx4 lacc = {0.f, 0.f, 0.f, 0.f};
  intx8 ones_a;
  {
    const int one = (lane == 0 || lane == 32 || lane == 20 || lane == 52) ? 0x38383838 : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones_a[e] = one;
  }

  const int n_kv_all = (N + T::BN - 1) / T::BN;
  const int n_kv = CAUSAL ? min(n_kv_all, (q0 + T::BM + T::BN - 1) / T::BN) : n_kv_all;
  const int n_wave = CAUSAL ? min(n_kv, (wave_q_lo + T::QW - 1) / T::BN + 1) : n_kv;

  // ---- producers: one 16-byte LDS-DMA per lane per tile ---------------------
  // LDS chunk x = 64 * wave + lane of a tile; row r = x / 8 holds, for K, key
  // key_of_row(r % 32) of its 32-row block.
  int k_src, v_src;
  {
    const int x = 64 * wave + lane;
    const int r = x >> 3, pos = x & 7;
    k_src = ((r & ~31) | key_of_row(r & 31)) * D + 16 * (pos ^ fp8_k_swz(r));
    v_src = r * D + 16 * (pos ^ fp8_v_swz(r));
  }
  // Every interval issues one K and one V load per wave (the waits count
  // them). With Q staging, K loads past the sequence go to the junk line.
  auto fetch_k = [&](int j) __attribute__((always_inline)) {
    load16_to_lds(rk, j * T::TILE_BYTES + k_src,
                  (STAGE_Q && j >= n_kv) ? (lds_char*)smem_raw + T::JUNK_OFFSET
                                         : k_ring + (j % T::SLOTS) * T::TILE_BYTES + wave * 1024);
  };
  // The next tile's Q rows, this wave's share, into the K ring; without a
  // next tile the loads read past the buffer (zeros), so the count is fixed.
  auto fetch_q_next = [&]() __attribute__((always_inline)) {
    const int tn = t_next < 0 ? t : t_next;
    const int bh_n = tn / p.n_qt;
    const int qt_n = tn - bh_n * p.n_qt;
    const __amdgpu_buffer_rsrc_t rq_n = make_rsrc(p.q + (size_t)bh_n * (size_t)N * D, head_bytes);
    const int off = t_next < 0 ? 0x7ffffff0 - 128 : (qt_n * T::BM + wave * T::QW + l32) * D + 32 * hh;
#pragma unroll
    for (int i = 0; i < T::Q_LOADS; ++i)
      load16_to_lds(rq_n, off + 64 * (i >> 1) + 16 * (i & 1), k_ring + wave * T::Q_LOADS * 1024 + 1024 * i);
  };
  auto fetch_v = [&](int j) __attribute__((always_inline)) {
    load16_to_lds(rv, j * T::TILE_BYTES + v_src,
                  v_ring + (j % T::SLOTS) * T::TILE_BYTES + wave * 1024);
  };

  // ---- consumer-side LDS offsets --------------------------------------------
  // K (A of T): row l32 of block kb, chunks 4 s + 2 hh and + 1.
  int k_rd[T::KSTEPS][2];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s)
#pragma unroll
    for (int e = 0; e < 2; ++e) k_rd[s][e] = l32 * D + 16 * ((4 * s + 2 * hh + e) ^ fp8_k_swz(l32));
  constexpr int K_BLOCK_BYTES = 32 * D;
  // V^T (A of U), d block b: source lane s16 of 16-lane group g reads 8 bytes
  // of key 16 rho + 8 hh + s16 / 2 at d = 32 b + 16 (g % 2) + 8 (s16 % 2);
  // run rho adds 16 rows.
  int v_rd[T::DBLK];
  {
    const int s16 = lane & 15, g = lane >> 4;
    const int key = 8 * hh + (s16 >> 1);
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b)
      v_rd[b] = key * D + 16 * ((2 * b + (g & 1)) ^ fp8_v_swz(key)) + 8 * (s16 & 1);
  }
  constexpr int V_RUN_BYTES = 16 * D;

  floatx16 sacc[T::KB];  // S_j^T (fp32)
  intx8 pf;              // P_j^T in E4M3: B operand of U_j

  auto k_operand = [&](const lds_char* ks, int kb, int s) __attribute__((always_inline)) {
    const intx4 a = *(const lds_intx4*)(ks + k_rd[s][0] + kb * K_BLOCK_BYTES);
    const intx4 b = *(const lds_intx4*)(ks + k_rd[s][1] + kb * K_BLOCK_BYTES);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto v_operand = [&](const lds_char* vs, int b) __attribute__((always_inline)) {
    intx2 r[T::RUNS];
#pragma unroll
    for (int rho = 0; rho < T::RUNS; ++rho)
      r[rho] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2*)(vs + v_rd[b] + rho * V_RUN_BYTES));
    return intx8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };

  const float c2 = p.scale_log2;

  auto mask_tile = [&](int j) __attribute__((always_inline)) {
    const int j0 = j * T::BN;
    if ((j0 + T::BN > N) || (CAUSAL && j0 + T::BN - 1 > wave_q_lo)) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
          if (key >= N || (CAUSAL && key > qrow)) sacc[kb][i] = -INFINITY;
        }
    }
  };
  // P_j^T in E4M3: byte j = 16 kb + i of pf is 2^(s c2 - m_run) of register i
  // of block kb.
  // Packing: v_cvt_pk_fp8_f32 writes one 16-bit half of its destination and
  // keeps the other, taken from its `old` operand. The high half is written
  // by the second conversion, so in the vector interval the first one's
  // `old` is a value that dies there (its first input): with 0 the compiler
  // zeroed a register first, one extra instruction per packed word. cvt_hi,
  // in the matrix-core interval, keeps 0: in place there, the packed words
  // would sit in the registers of the accumulator the next T MFMAs rewrite
  // (measured 0.3% slower).
  auto exp_pack = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, i = 4 * (w & 3);
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i + u], c2, -m_run));
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], __builtin_bit_cast(int, e[0]), false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], x, true);
    }
  };
  // Fast-pass split of exp_pack: in the vector interval, key block 0's
  // weights are packed and block 1's are left in place in sacc[1] as fp32;
  // the matrix-core interval packs them (cvt_hi) while its first two MFMAs,
  // which rewrite only sacc[0], run. The packed bytes are the same.
  auto exp_pack_lo = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 4 * w;
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[0][i + u], c2, -m_run));
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], __builtin_bit_cast(int, e[0]), false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], x, true);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[1][i], c2, -m_run));
  };
  auto cvt_hi = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int w = 4; w < 8; ++w) {
      const int i = 4 * (w & 3);
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[1][i], sacc[1][i + 1], 0, false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[1][i + 2], sacc[1][i + 3], x, true);
    }
  };
  auto tile_max = [&]() __attribute__((always_inline)) {
    float t[11];
#pragma unroll
    for (int k = 0; k < 10; ++k) {
      const int a = 3 * k;
      t[k] = max3(sacc[a >> 4][a & 15], sacc[(a + 1) >> 4][(a + 1) & 15], sacc[(a + 2) >> 4][(a + 2) & 15]);
    }
    t[10] = max3(sacc[1][14], sacc[1][15], sacc[1][15]);
    const float u0 = max3(t[0], t[1], t[2]), u1 = max3(t[3], t[4], t[5]);
    const float u2 = max3(t[6], t[7], t[8]), u3 = max3(t[9], t[10], t[10]);
    const float mx = max3(max3(u0, u1, u2), u3, u3);
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return max3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1])) * c2;
  };
  // C stage for key tile j: weights against the current reference, the row
  // max alongside; the reference moves (and O, l are rescaled and the
  // weights formed again) only when a row's max grows by more than
  // 2^RESCALE_LOG2, so every weight stays <= 256.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    mask_tile(j);
    exp_pack();
    asm volatile("" : "+v"(pf));
    const float m_tile = tile_max();
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + RESCALE_LOG2) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc *= alpha;
#pragma unroll
      for (int b = 0; b < T::DBLK; ++b) oacc[b] *= alpha;
      exp_pack();
    }
  };
  // Fast C stage: weights against the fixed reference, no row max; block
  // 1's weights are packed in the next matrix-core interval.
  auto softmax_fast = [&](int j) __attribute__((always_inline)) {
    mask_tile(j);
    exp_pack_lo();
  };
  // Tile 0 of the fast pass: the reference is the tile's row max.
  auto softmax_first_fast = [&]() __attribute__((always_inline)) {
    mask_tile(0);
    m_run = tile_max();
    exp_pack_lo();
  };
  // T stage alone (tile 0): S^T = K_0 Q^T.
  auto qk = [&]() __attribute__((always_inline)) {
    const lds_char* ks = k_ring;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      sacc[kb] = mfma_fp8(k_operand(ks, kb, 0), qf[0], floatx16{});
      sacc[kb] = mfma_fp8(k_operand(ks, kb, 1), qf[1], sacc[kb]);
    }
  };
  // U stage alone (last tile of a wave).
  auto pv = [&](int j, auto split_tag) __attribute__((always_inline)) {
    if constexpr (decltype(split_tag)::value) cvt_hi();
    const lds_char* vs = v_ring + (j % T::SLOTS) * T::TILE_BYTES;
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b) oacc[b] = mfma_fp8(v_operand(vs, b), pf, oacc[b]);
    lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones_a, pf, lacc, 0, 0, 0, 127, 0, 127);
  };
  // Matrix-core interval of iteration j: U_{j-1} and T_j, then the row sum
  // of P_{j-1}. Exact pass: U and T alternate. Fast pass (SPLIT): T_j's two
  // MFMAs of key block 0 first, then the packing of P_{j-1}'s block 1
  // (cvt_hi), then the four U MFMAs and T_j's block 1. Each operand is read
  // AHEAD MFMAs before its use. The reads are inline asm: the compiler would
  // otherwise wait for every LDS-DMA in flight (vmcnt(0)) before them, though
  // none targets the slots read here. Their completion is waited for
  // explicitly: LDS reads finish in order, so before MFMA i only the reads
  // of operands i+1 .. i+AHEAD may be outstanding.
  auto mfma_interval = [&](auto u_tag, auto split_tag) __attribute__((always_inline)) {
    constexpr int U = decltype(u_tag)::value;
    constexpr bool SPLIT = decltype(split_tag)::value;
    constexpr int PREV = (U + T::SLOTS - 1) % T::SLOTS;
    constexpr int NPV = T::DBLK, NT = T::KB * T::KSTEPS;
    static_assert(NPV == 4 && NT == 4, "four U and four T MFMAs");
    constexpr int NM = NPV + NT, AHEAD = 2;
    constexpr int K_OFF = U * T::TILE_BYTES;
    constexpr int V_OFF = T::SLOTS * T::TILE_BYTES + PREV * T::TILE_BYTES;
    const uint32_t base = (uint32_t)(uintptr_t)k_ring;
    // slot i: a U MFMA (d block idx(i)) or a T MFMA (n = idx(i): key block
    // n / 2, k-step n % 2)
    auto is_u = [](int i) constexpr { return SPLIT ? (i >= 2 && i < 6) : (i & 1) == 0; };
    auto idx = [](int i) constexpr { return SPLIT ? (i < 2 ? i : (i < 6 ? i - 2 : i - 4)) : i >> 1; };
    auto reads = [is_u](int i) constexpr { return is_u(i) ? T::RUNS : 2; };
    auto operand = [&](auto i_tag) __attribute__((always_inline)) {
      constexpr int i = decltype(i_tag)::value;
      constexpr int n = idx(i);
      intx8 r;
      if constexpr (is_u(i)) {
        intx2 x[T::RUNS];
#pragma unroll
        for (int rho = 0; rho < T::RUNS; ++rho)
          asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2"
                       : "=v"(x[rho])
                       : "v"(base + v_rd[n]), "i"(V_OFF + rho * V_RUN_BYTES));
        r = intx8{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
      } else {
        constexpr int kb = n >> 1, st = n & 1;
        intx4 a, b;
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a) : "v"(base + k_rd[st][0]), "i"(K_OFF + kb * K_BLOCK_BYTES));
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(b) : "v"(base + k_rd[st][1]), "i"(K_OFF + kb * K_BLOCK_BYTES));
        r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      return r;
    };
    intx8 ring[AHEAD];
    ring[0] = operand(std::integral_constant<int, 0>{});
    ring[1] = operand(std::integral_constant<int, 1>{});
    auto step = [&](auto i_tag) __attribute__((always_inline)) {
      constexpr int i = decltype(i_tag)::value;
      __builtin_amdgcn_sched_barrier(0);
      intx8 a = ring[i % AHEAD];
      if constexpr (i + AHEAD < NM) ring[i % AHEAD] = operand(std::integral_constant<int, i + AHEAD>{});
      constexpr int after = (i + 1 < NM ? reads(i + 1) : 0) + (i + 2 < NM ? reads(i + 2) : 0);
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(after));
      constexpr int n = idx(i);
      // the empty asm keeps each MFMA in this interval (LLVM would sink the
      // U MFMAs, whose results are not needed until the next interval)
      if constexpr (is_u(i)) {
        oacc[n] = mfma_fp8(a, pf, oacc[n]);
        asm volatile("" : "+v"(oacc[n]));
      } else {
        constexpr int kb = n >> 1, st = n & 1;
        sacc[kb] = mfma_fp8(a, qf[st], st == 0 ? floatx16{} : sacc[kb]);
        asm volatile("" : "+v"(sacc[kb]));
      }
      if constexpr (SPLIT && i == 1) {
        __builtin_amdgcn_sched_barrier(0);
        cvt_hi();
      }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
    static_assert(NM == 8, "eight MFMAs per interval");
    lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones_a, pf, lacc, 0, 0, 0, 127, 0, 127);
    asm volatile("" : "+v"(lacc));
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- ping-pong schedule (as the FP16 kernel) ------------------------------
  // Rings (slot = tile % 4). K_t: DMA issued in local interval 2t-5, waited
  // for at the end of local 2t-2, read in global 2t .. 2t+1. V_t: DMA issued
  // in local 2t-3, waited for at the end of local 2t, read in global 2t+2 ..
  // 2t+3. The next DMA into either slot is issued at local 2t+3 or later.
  auto sync = [&]() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
  auto mfma_sync = [&]() __attribute__((always_inline)) {
    // everything but the two DMAs of the latest vector interval has landed
    asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
  };
  auto vector_sync = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto produce_issue = [&](int j) __attribute__((always_inline)) {
    fetch_k(j + 3);
    fetch_v(j + 2);
  };
  auto steady = [&](int j, auto u_tag, auto exact_tag) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    mfma_interval(u_tag, std::integral_constant<bool, !decltype(exact_tag)::value>{});
    __builtin_amdgcn_s_setprio(0);
    mfma_sync();
    produce_issue(j);
    if constexpr (decltype(exact_tag)::value) softmax(j);
    else softmax_fast(j);
    vector_sync();
  };
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;
  using U3 = std::integral_constant<int, 3>;

  // The whole K/V pipeline; the fast variant forms no row max after tile 0.
  auto run_pipeline = [&](auto exact_tag) __attribute__((always_inline)) {
    fetch_k(0);
    fetch_k(1);
    fetch_k(2);
    fetch_v(0);
    fetch_v(1);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (group == 1) sync();

    // j = 0: T_0, then C_0 (exact: it sets the reference)
    if (n_wave > 0) qk();
    mfma_sync();
    produce_issue(0);
    if (n_wave > 0) {
      if constexpr (decltype(exact_tag)::value) softmax(0);
      else softmax_first_fast();
    }
    vector_sync();
    int j = 1;
    for (; j + 4 <= n_wave; j += 4) {
      steady(j, U1{}, exact_tag);
      steady(j + 1, U2{}, exact_tag);
      steady(j + 2, U3{}, exact_tag);
      steady(j + 3, U0{}, exact_tag);
    }
    if (j < n_wave) {
      steady(j, U1{}, exact_tag);
      ++j;
      if (j < n_wave) {
        steady(j, U2{}, exact_tag);
        ++j;
        if (j < n_wave) {
          steady(j, U3{}, exact_tag);
          ++j;
        }
      }
    }
    // n_wave <= j <= n_kv: the last U for this wave, then idle intervals in
    // which the wave still loads its share of the workgroup's tiles
    for (; j <= n_kv; ++j) {
      if (j == n_wave && j >= 1) pv(j - 1, std::integral_constant<bool, !decltype(exact_tag)::value>{});
      mfma_sync();
      produce_issue(j);
      // every wave is past its last T stage (group 1's reads end one
      // interval earlier), so the K ring is idle from here on
      if (STAGE_Q && j == n_kv) fetch_q_next();
      vector_sync();
    }
    if (group == 0) sync();
    // every DMA but the staged Q loads has landed in every wave: the V ring
    // (and the O staging beyond it) may be reused
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(STAGE_Q ? T::Q_LOADS : 0) : "memory");
  };
  // true in every wave if `mine` holds in some lane of some wave. The flags
  // sit in the V ring (idle after the pipeline's last wait; the K ring may
  // be receiving the next tile's Q).
  auto any_wave = [&](bool mine) __attribute__((always_inline)) {
    const bool bad = __builtin_amdgcn_ballot_w64(mine) != 0;
    sync();
    __attribute__((address_space(3))) int* flags = (__attribute__((address_space(3))) int*)v_ring;
    if (lane == 0) flags[wave] = bad ? 1 : 0;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    int any = 0;
#pragma unroll
    for (int w = 0; w < T::WAVES; ++w) any |= flags[w];
    any = __builtin_amdgcn_readfirstlane(any);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    return any != 0;
  };
  if (!CAUSAL) {
    run_pipeline(std::integral_constant<bool, CAUSAL>{});
    // A weight that overflowed E4M3 is NaN, and so is its row sum.
    if (any_wave(!(sum_halves(lacc[0]) < INFINITY))) {
      // the staged Q for the next tile is landing in the K ring, which the
      // rerun refills (and stages again at its end)
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int b = 0; b < T::DBLK; ++b) oacc[b] = floatx16{};
      lacc = floatx4{};
      m_run = -INFINITY;
      run_pipeline(std::true_type{});
    }
  } else {
    run_pipeline(std::true_type{});
  }

  // ---- epilogue: O = descale_v O_acc / l, lse = (m + log2 l) ln 2 ---------------
  // register i of block b holds d = 32 b + 8 (i / 4) + 4 hh + i % 4
  // O goes through LDS so that the global stores are whole rows (as in the
  // FP16 kernel): each wave stages its 32 rows from the start of the V ring,
  // rows padded by 16 bytes, and stores 16 bytes per lane, 16 lanes per row,
  // by raw-buffer stores (rows past N out of range): exactly EPI_STORES per
  // wave, which the next tile's wait for its staged Q counts on.
  const float l_tot = sum_halves(lacc[0]);
  const float f = p.descale_v / l_tot;
  constexpr int O_STRIDE = T::O_STRIDE;
  lds_char* const ob = v_ring + wave * T::QW * O_STRIDE;
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      half4 w = {(_Float16)(oacc[b][4 * g + 0] * f), (_Float16)(oacc[b][4 * g + 1] * f),
                 (_Float16)(oacc[b][4 * g + 2] * f), (_Float16)(oacc[b][4 * g + 3] * f)};
      *(__attribute__((address_space(3))) half4*)(ob + l32 * O_STRIDE + (32 * b + 8 * g + 4 * hh) * 2) = w;
    }
  constexpr int LANES_PER_ROW = D / 8;
  constexpr int ROWS_PER_STORE = 64 / LANES_PER_ROW;
  static_assert(T::QW / ROWS_PER_STORE + 1 == T::EPI_STORES, "epilogue store count");
  const int srow = lane / LANES_PER_ROW, scol = 8 * (lane % LANES_PER_ROW);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + head, head_bytes * 2u);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + (size_t)bh * N, (uint32_t)N * 4u);
#pragma unroll
  for (int r0 = 0; r0 < T::QW; r0 += ROWS_PER_STORE) {
    const int row = r0 + srow;
    const half8 x = *(const __attribute__((address_space(3))) half8*)(ob + row * O_STRIDE + 2 * scol);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(intx4, x), ro,
                                           ((wave_q_lo + row) * D + scol) * 2, 0, 0);
  }
  const float lse_v = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(lse_v), rl, hh == 0 ? qrow * 4 : 0x7ffffff0, 0, 0);
  // the next tile's DMAs may refill the V ring only once every wave has read
  // its staged rows back
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Persistent, with the FP16 kernel's tile schedule: one workgroup per CU (a
// multiple of 8) or one per tile, odd passes reversed within each XCD.
template <bool CAUSAL>
__global__ __launch_bounds__(Fp8Tile::THREADS, 1) void fmha_fwd_fp8_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Fp8Tile::LDS_BYTES];
  const int G = p.total_wg;
  auto tile_of = [&](int r) { return persistent_tile(r, G); };
  for (int r = 0;; ++r) {
    const int t = tile_of(r);
    if (t < 0) break;
    fwd_fp8_tile<CAUSAL>(p, t, tile_of(r + 1), r > 0, smem_raw);
  }
  // a non-causal workgroup's last tile staged Q loads past the buffer
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace fmha
