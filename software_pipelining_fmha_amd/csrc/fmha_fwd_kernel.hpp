// Fused multi-head attention forward pass for gfx950 (MI355X, CDNA4).
//
// The kernel is persistent: one workgroup per CU walks the (batch, head,
// query tile) tiles, one at a time. Per tile the query rows stay in VGPRs.
// Key/value tiles stream from HBM into LDS rings by LDS-DMA. Each stage of
// the pages maps onto gfx950 units:
// - T stage, S = Q K^T (Tawa, section III-D): fp16 MFMA, fp32 accumulate;
// - C stage, online softmax with rescale (PipeThreader's softmax and
//   rescale tasks): VALU, exp2 on the transcendental unit;
// - U stage, O += P V: fp16 MFMA.
//
// Register layouts (one 64-lane wave):
// * Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_f16. A lane of the accumulator then holds 16 keys of
//   one query column. So the row max is an in-lane reduction plus one swap
//   between the two 32-lane halves.
// * Key rows are written to LDS under a permutation that swaps bits 2 and 3
//   of the row index within each 32-row block. With it, accumulator register
//   i of lane-half h holds key 16*(i/8) + 8*h + i%8. Eight consecutive
//   registers therefore cover 8 consecutive keys. After conversion to fp16
//   they are the B operand of O^T += V^T P^T, with no shuffle.
// * V stays in natural [key][d] layout in LDS. The A operand of the U stage
//   (eight consecutive keys of one d column per lane) comes from two
//   ds_read_b64_tr_b16, each returning four keys of one column per lane.
// * O^T accumulates with one query per lane column. The per-row rescale
//   factor is therefore a per-lane scalar.
// * Row sums of P run on the matrix core as well (one 16x16x32 MFMA per PV
//   k-step), so the vector ALU only forms the weights.
//
// Exponent reference: softmax is the same for any per-row offset, and the
// running max only keeps the weights in range. So after the first key tile
// the C stage keeps that tile's row max as a fixed reference and forms no
// row max at all. If a later score exceeds the reference by 16 (base 2), its
// weight overflows fp16 and the row sum turns non-finite. The workgroup then
// recomputes its tile with the running max and lazy rescale, so every
// output is the exact-path output in that case. The causal kernel runs the
// exact pass only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fmha {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// Reference-max slack (base 2) before O and l are rescaled; every weight
// then stays at or below 2^slack. The FP16 kernel takes 15: fp16 holds up
// to 65504, and on sharp rows a wider slack means fewer rescales. The FP8
// kernel takes 8, since E4M3 holds no more than 448.
constexpr float RESCALE_LOG2_F16 = 15.0f;
constexpr float RESCALE_LOG2 = 8.0f;
// MFMA slots by which an LDS operand read precedes its MFMA.
constexpr int OPERAND_AHEAD = 4;
// U MFMAs at the head of a matrix-core interval (T MFMAs close it).
constexpr int LEAD_U = 2;

struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;
  int N;            // sequence length (queries = keys)
  int n_qt;         // query tiles per head
  int total_wg;     // B * H * n_qt
  float scale_log2; // |scale| * log2(e) (> 0): scores go to the base-2 domain
  int q_sign;       // sign of scale (1, -1 or 0), folded into the Q operand
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
  static constexpr int TILE_BYTES = BN * D * 2; // one K or V tile in LDS
  static constexpr int SLOTS = 4;               // ring depth for K and for V
  static constexpr int RING_BYTES = SLOTS * TILE_BYTES;
  // O is staged from the start of the V ring, rows padded by 16 bytes
  static constexpr int O_STRIDE = D * 2 + 16;
  static constexpr int O_STAGE_BYTES = WAVES * QW * O_STRIDE;
  static constexpr int LDS_BYTES = RING_BYTES + O_STAGE_BYTES;
  // The next tile's Q goes to the K ring, once per wave: KSTEPS loads of
  // 1 KB, load s holding every lane's k-step-s operand in lane order.
  static_assert(WAVES * KSTEPS * 1024 == RING_BYTES, "one Q tile fills the K ring");
  // VMEM instructions of the epilogue, per wave: O rows and lse
  static constexpr int EPI_STORES = QW * D * 2 / 1024 + 1;
  // one tile = TILE_BYTES / 1024 wave-wide 16-byte-per-lane LDS-DMA loads
  static constexpr int LOADS_PER_TILE = TILE_BYTES / 1024;
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TILE / WAVES;  // per tile
  static_assert(LOADS_PER_TILE % WAVES == 0 && LOADS_PER_WAVE >= 1, "tile loads split over waves");
  static_assert(LDS_BYTES <= 160 * 1024, "fits the CU's LDS");
  static_assert(O_STAGE_BYTES >= RING_BYTES, "the V ring lies inside the O staging");
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

// x plus the partner lane's x (lane ^ 32), via v_permlane32_swap. After the
// swap the two results hold {x[l], x[l^32]} in some order; the sum is
// symmetric, so every lane gets the same value.
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(a, b, c) in one instruction. Scores are never NaN here (MFMA results or
// -inf from masking), so no quieting of the inputs is needed, which fmaxf
// would add in IEEE mode.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Key held by row p of an LDS K tile: bits 2 and 3 of p swapped (an involution).
__device__ __forceinline__ int key_of_row(int p) {
  const int flip = ((p >> 2) ^ (p >> 3)) & 1;
  return p ^ (flip * 0xC);
}

// Chunk swizzle of row p of a K tile. 16 lanes reading one chunk column of
// 16 consecutive rows must hit 16 distinct 4-bank groups of the 64 banks: at
// d = 128 a row is 256 bytes (every bank once), so the 16 rows need 16
// distinct chunks; at d = 64 a row is 128 bytes (half the banks, by the
// row's parity), so each parity's 8 rows need 8 distinct chunks.
template <int D>
__device__ __forceinline__ int k_swz(int p) {
  return D == 128 ? (p & 15) : ((p >> 1) & 7);
}
// LDS byte offset of 16-byte chunk c of row p in a K tile.
template <int D>
__device__ __forceinline__ int k_chunk_off(int p, int c) {
  constexpr int CPR = D / 8;
  return (p * CPR + (c ^ k_swz<D>(p))) * 16;
}

// Staged Q rows -> registers: k-step s of lane l sits at base + 1024 s + 16 l.
// One asm block issues every read and waits for them, so no output register
// is taken as written before its data has landed.
template <int KSTEPS>
__device__ __forceinline__ void read_staged_q(uint32_t base, half8 (&qf)[KSTEPS]);
template <>
__device__ __forceinline__ void read_staged_q<8>(uint32_t base, half8 (&qf)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3]), "=&v"(qf[4]), "=&v"(qf[5]),
        "=&v"(qf[6]), "=&v"(qf[7])
      : "v"(base)
      : "memory");
}
template <>
__device__ __forceinline__ void read_staged_q<4>(uint32_t base, half8 (&qf)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3])
      : "v"(base)
      : "memory");
}

// Tile t. Non-causal: t_next is the tile this workgroup runs next (-1:
// none); once the last T stage is done, its Q rows go to the K ring by
// LDS-DMA, and with q_staged the next call takes its Q from there instead of
// from HBM, where every workgroup of the chip would request its Q at the
// same moment (equal tiles turn over together). Causal tiles differ in
// length and turn over at different times; staging measured slower there,
// so the causal kernel loads Q at the tile's start.
template <int D, bool CAUSAL>
// `wave` is the caller's (uniform) wave index. In the non-causal kernel the
// lane index is formed anew in every tile by an asm mbcnt the compiler
// cannot hoist: otherwise it hoists every lane-derived constant out of the
// tile loop, spills them (that kernel holds both passes and runs at 256
// VGPRs), and each reload, a vector-memory load, waits for the previous
// tile's stores. The causal kernel has the registers to keep them.
__device__ __forceinline__ void fwd_tile(const Params& p, int t, int t_next, bool q_staged,
                                         int wave, char* smem_raw) {
  using T = Tile<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* const k_ring = (lds_char*)smem_raw;
  lds_char* const v_ring = k_ring + T::SLOTS * T::TILE_BYTES;

  int lane;
  if constexpr (CAUSAL)
    lane = threadIdx.x & 63;
  else
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int group = wave >> 2;  // waves w and w + 4 share a SIMD
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work decomposition -------------------------------------------------
  // Tile id t -> (b*H + h, query tile). The persistent loop below hands one
  // XCD consecutive ids, i.e. the query tiles of one head, so they share its
  // L2 copy of that head's K and V.
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
  const uint32_t q_stage = (uint32_t)(uintptr_t)k_ring + wave * T::KSTEPS * 1024;
  constexpr bool STAGE_Q = !CAUSAL;
  if (STAGE_Q && q_staged) {
    // The previous tile staged this wave's rows, and its epilogue's
    // EPI_STORES stores are the only vector-memory operations since: once
    // those older loads have landed in every wave, the rows are read, and a
    // barrier keeps the K ring from being refilled before every wave has.
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(T::EPI_STORES) : "memory");
    // the lane offset is formed here, in asm the compiler cannot merge with
    // `lane`: a register live from the tile's start may be spilled, and its
    // reload (a vector-memory load) would wait for the epilogue's stores
    uint32_t lane16;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 4, %0"
                 : "=v"(lane16));
    read_staged_q<T::KSTEPS>(q_stage + lane16, qf);
    asm volatile("s_barrier" ::: "memory");
  } else {
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s)
      qf[s] = __builtin_bit_cast(half8, load16(rq, (qrow * D + 16 * s + 8 * hh) * 2));
  }
  // The C stage needs a positive multiplier (its row max is taken on the raw
  // scores, and masked scores are -inf). So the sign of scale rides on Q,
  // where multiplying by -1 or 0 is exact: (-q).k * |scale| = q.k * scale,
  // and scale = 0 gives scores of exactly 0 (uniform weights).
  if (p.q_sign != 1) {
    const _Float16 f = (_Float16)(float)p.q_sign;
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s) qf[s] = qf[s] * f;
  }

  floatx16 oacc[T::DBLK];
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -INFINITY;  // reference max of scaled scores (base-2 domain)
  // Row sums of P on the matrix core: v_mfma_f32_16x16x32_f16 with a 0/1 A
  // operand and P^T_j (as laid out for the 32x32x16 U MFMA) as B. Read as a
  // 16x16x32 operand, lane l of that B holds keys 8*(l/32) .. +7 of query
  // 16*((l/16)%2) + l%16. A row 0 selects the key groups of queries 0..15
  // (lanes 0, 32), A row 4 those of queries 16..31 (lanes 20, 52). Register 0
  // of lane q < 32 of the accumulator then holds the row sum of query q; every
  // other element stays 0. The sum adds exactly the fp16 weights of U, in fp32.
  floatx4 lacc = {0.f, 0.f, 0.f, 0.f};
  half8 ones_a;
  {
    const _Float16 one = (lane == 0 || lane == 32 || lane == 20 || lane == 52) ? (_Float16)1.f : (_Float16)0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones_a[e] = one;
  }

  const int n_kv_all = (N + T::BN - 1) / T::BN;
  const int n_kv = CAUSAL ? min(n_kv_all, (q0 + T::BM + T::BN - 1) / T::BN) : n_kv_all;
  // Tiles this wave computes: causal rows see no key past wave_q_lo + 31.
  const int n_wave = CAUSAL ? min(n_kv, (wave_q_lo + T::QW - 1) / T::BN + 1) : n_kv;

  // ---- producers ---------------------------------------------------------------
  // K and V: HBM -> LDS ring slots by LDS-DMA, no register staging. Wave w
  // issues loads w*LOADS_PER_WAVE .. +LOADS_PER_WAVE-1 of a tile; load i
  // fills the tile's LDS chunks 64*i .. 64*i+63 (one per lane), and each lane
  // fetches the global chunk that the swizzled layout puts there. Both rings
  // have SLOTS slots (slot = tile % SLOTS).
  int k_src[T::LOADS_PER_WAVE];
#pragma unroll
  for (int r = 0; r < T::LOADS_PER_WAVE; ++r) {
    const int x = 64 * (wave * T::LOADS_PER_WAVE + r) + lane;  // LDS chunk index
    const int row = x / T::CPR, slot = x % T::CPR;
    k_src[r] = (key_of_row(row) * D + 8 * (slot ^ k_swz<D>(row))) * 2;
  }
  auto fetch_k = [&](int j) __attribute__((always_inline)) {
    lds_char* dst = k_ring + (j % T::SLOTS) * T::TILE_BYTES + wave * T::LOADS_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i)
      load16_to_lds(rk, j * T::BN * D * 2 + k_src[i], dst + i * 1024);
  };
  // V stays in natural [key][d] layout; chunk c of key row k is stored at
  // chunk c ^ v_swz(k), so that the transposing operand reads below touch
  // distinct banks.
  auto v_swz = [](int row) __attribute__((always_inline)) {
    return ((D == 128 ? 4 : 2) * (row & 3)) % T::CPR;
  };
  int v_src[T::LOADS_PER_WAVE];
#pragma unroll
  for (int r = 0; r < T::LOADS_PER_WAVE; ++r) {
    const int x = 64 * (wave * T::LOADS_PER_WAVE + r) + lane;
    const int row = x / T::CPR, pos = x % T::CPR;
    v_src[r] = (row * D + 8 * (pos ^ v_swz(row))) * 2;
  }
  auto fetch_v = [&](int j) __attribute__((always_inline)) {
    lds_char* dst = v_ring + (j % T::SLOTS) * T::TILE_BYTES + wave * T::LOADS_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i)
      load16_to_lds(rv, j * T::BN * D * 2 + v_src[i], dst + i * 1024);
  };

  // ---- consumer-side LDS addresses (per lane, constant over the loop) --------
  // The operand reads are inline asm with explicit lgkmcnt waits: as
  // builtins, the compiler would wait for every LDS-DMA in flight (vmcnt(0))
  // before them, though none targets the slots read. Each address is a lane
  // register plus an immediate (slot, key block, k-step).
  // QK^T A operand: row 32*kb + l32 of the K tile, chunk 2*s + hh. The
  // swizzle depends on the row only through its low 4 bits, so the 32-row
  // block kb adds a constant.
  uint32_t k_rd[T::KSTEPS];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s)
    k_rd[s] = (uint32_t)(uintptr_t)k_ring + k_chunk_off<D>(l32, 2 * s + hh);
  constexpr int K_BLOCK_BYTES = 32 * T::CPR * 16;
  // PV A operand (d block b, k-step st): lane l needs d = 32b + l % 32 of
  // keys 16st + 8hh .. +7, eight keys of one V column: two ds_read_b64_tr_b16
  // of four keys each. In 16-lane group g, source lane s reads the four d
  // values 32b + 16(g % 2) + 4(s % 4) .. +3 of key 16st + 8hh + 4r + s / 4
  // (read r = 0, 1); result lane i of the group then holds d
  // 32b + 16(g % 2) + i of those four keys. The key's low two bits are s / 4
  // whatever st and r are, so the swizzle is fixed per lane and d block.
  uint32_t v_rd[T::DBLK];
  {
    const int s16 = lane & 15, g = lane >> 4;
    const int key = 8 * hh + (s16 >> 2);
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b) {
      const int c = 4 * b + 2 * (g & 1) + ((s16 & 3) >> 1);
      v_rd[b] = (uint32_t)(uintptr_t)v_ring + key * D * 2 + 16 * (c ^ v_swz(key)) + 8 * (s16 & 1);
    }
  }
  constexpr int V_R_BYTES = 4 * D * 2;    // read r = 1: four keys on
  constexpr int V_ST_BYTES = 16 * D * 2;  // next k-step: sixteen keys on

  floatx16 sacc[T::KB];   // S_j^T (fp32)
  half8 pf[T::PSTEPS];    // P_j^T in fp16: B operand of PV_j
  // Row sums of P_j for PV k-step st.
  auto row_sum = [&](int st) __attribute__((always_inline)) {
    lacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones_a, pf[st], lacc, 0, 0, 0);
  };

  // Operand reads (issue only; the caller waits). A T operand is one
  // ds_read_b128, a U operand two ds_read_b64_tr_b16.
  auto read_t = [&](auto slot_tag, int n) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    const int kb = n % T::KB, st = n / T::KB;
    half8 a;
    asm volatile("ds_read_b128 %0, %1 offset:%2"
                 : "=v"(a)
                 : "v"(k_rd[st]), "i"(SLOT * T::TILE_BYTES + kb * K_BLOCK_BYTES));
    return a;
  };
  auto read_u = [&](auto slot_tag, int n) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    const int st = n / T::DBLK, b = n % T::DBLK;
    shortx4 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(lo)
                 : "v"(v_rd[b]), "i"(SLOT * T::TILE_BYTES + st * V_ST_BYTES));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(hi)
                 : "v"(v_rd[b]), "i"(SLOT * T::TILE_BYTES + st * V_ST_BYTES + V_R_BYTES));
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // T stage of key tile 0 alone: S^T = K_0 Q^T.
  auto qk = [&]() __attribute__((always_inline)) {
    using S0 = std::integral_constant<int, 0>;
#pragma unroll
    for (int st = 0; st < T::KSTEPS; ++st) {
      half8 a[T::KB];
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) a[kb] = read_t(S0{}, st * T::KB + kb);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[T::KB - 1]));
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[kb], qf[st], st == 0 ? floatx16{} : sacc[kb],
                                                          0, 0, 0);
    }
  };
  // U stage of a wave's last key tile alone: O^T += V^T P^T, V in `slot`.
  auto pv = [&](auto slot_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < T::PSTEPS * T::DBLK; ++n) {
      half8 a = read_u(slot_tag, n);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a));
      const int st = n / T::DBLK, b = n % T::DBLK;
      oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[st], oacc[b], 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < T::PSTEPS; ++s) row_sum(s);
  };

  const float c2 = p.scale_log2;

  // C stage for key tile j. Keys past N (ragged tail) and, if causal, keys
  // after the query get score -inf.
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
  // P_j^T in fp16 (pf, the B operand of U_j): p = 2^(s*c2 - m_run).
  auto exp_pack = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < T::PSTEPS; ++st)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pf[st][i] = (_Float16)__builtin_amdgcn_exp2f(
            __builtin_fmaf(sacc[st >> 1][8 * (st & 1) + i], c2, -m_run));
  };
  // Row max of the masked scores (base-2 domain), as a shallow tree.
  auto tile_max = [&]() __attribute__((always_inline)) {
    // 32 scores: 11 + 4 + 2 + 1 max3, depth 4
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
  // C stage for key tile j. The weights are first formed against the current
  // reference max; the row max, computed alongside, only decides whether the
  // reference must move. It moves only when some row's max grows by more than
  // 2^RESCALE_LOG2_F16, so p <= 2^RESCALE_LOG2_F16 always. O and l share the
  // reference, so O / l is unchanged when it stays. When it moves, O and l
  // are rescaled (they hold every earlier tile here: U_{j-1} and its row sum
  // ran in the matrix-core interval before C_j) and the weights are formed
  // again from the scores, which are still intact.
  // Without the row max: the reference stays at tile 0's max. Weights stay
  // finite while no score exceeds it by 16 (base 2); past that they overflow
  // fp16, the row sum becomes inf, and the workgroup reruns the exact path.
  auto softmax_fast = [&](int j) __attribute__((always_inline)) {
    mask_tile(j);
    exp_pack();
  };
  auto softmax = [&](int j) __attribute__((always_inline)) {
    mask_tile(j);
    exp_pack();
    // the weights are formed here, before the branch, not inside it
#pragma unroll
    for (int st = 0; st < T::PSTEPS; ++st) asm volatile("" : "+v"(pf[st]));
    const float m_tile = tile_max();
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + RESCALE_LOG2_F16) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc *= alpha;  // lane q < 32 holds query q, as alpha does
#pragma unroll
      for (int b = 0; b < T::DBLK; ++b) oacc[b] *= alpha;
      exp_pack();
    }
  };
  // Matrix-core interval of a steady iteration: U_{j-1} (V slot (j-1) % 4)
  // and T_j (K slot j % 4), 2 * NPV MFMAs in a fixed order, plus the row-sum
  // MFMA after the last U MFMA of each k-step. Each operand is read
  // OPERAND_AHEAD slots before its MFMA; scheduling barriers keep that order,
  // and each MFMA waits (lgkmcnt) only for its own operand: LDS reads
  // complete in order, so the later operands' reads may still be pending.
  // Slot order: the first LEAD_U slots are U MFMAs, then T and U alternate,
  // and the last LEAD_U slots are T MFMAs. The operands of the first AHEAD
  // slots were read at the end of the wave's vector interval (K_j and V_{j-1}
  // are both visible by then). T slot n is key block n % KB at k-step n / KB and U slot n is d
  // block n % DBLK at k-step n / DBLK, so consecutive MFMAs never share an
  // accumulator.
  constexpr int NPV = T::PSTEPS * T::DBLK;
  constexpr int NM = 2 * NPV;
  static_assert(NPV == T::KSTEPS * T::KB, "as many U as T MFMAs");
  constexpr int AHEAD = OPERAND_AHEAD;
  static_assert(LEAD_U <= AHEAD && LEAD_U < NPV, "lead operands fit the read-ahead ring");
  // slot i -> (is U, index among its kind)
  auto slot_is_u = [](int i) constexpr {
    return i < LEAD_U ? true : (i >= NM - LEAD_U ? false : ((i - LEAD_U) & 1) == 1);
  };
  auto slot_n = [](int i) constexpr {
    return i < LEAD_U ? i : (i >= NM - LEAD_U ? i - NPV : (i - LEAD_U) / 2 + (((i - LEAD_U) & 1) ? LEAD_U : 0));
  };
  // LDS reads of slots i+1 .. i+AHEAD: those may still be outstanding when
  // slot i's operand has landed
  auto reads_after = [slot_is_u](int i) constexpr {
    int r = 0;
    for (int m = i + 1; m <= i + AHEAD && m < NM; ++m) r += slot_is_u(m) ? 2 : 1;
    return r;
  };
  static_assert([reads_after]() constexpr {
    int m = 0;
    for (int i = 0; i < NM; ++i) m = reads_after(i) > m ? reads_after(i) : m;
    return m;
  }() <= 15, "the wait count fits lgkmcnt");
  half8 ring[AHEAD];
  // End of a vector interval: the first AHEAD operands of the next
  // matrix-core interval (U_j from V slot j % 4, T_{j+1} from K slot
  // (j + 1) % 4), so that interval starts with its read-ahead ring full.
  auto prefetch_lead = [&](auto v_tag) __attribute__((always_inline)) {
    constexpr int KN = (decltype(v_tag)::value + 1) % 4;
#pragma unroll
    for (int i = 0; i < AHEAD; ++i)
      ring[i] = slot_is_u(i) ? read_u(v_tag, slot_n(i)) : read_t(std::integral_constant<int, KN>{}, slot_n(i));
  };
  auto mfma_interval = [&](auto k_tag, auto v_tag) __attribute__((always_inline)) {
    auto operand = [&](int i) __attribute__((always_inline)) {
      return slot_is_u(i) ? read_u(v_tag, slot_n(i)) : read_t(k_tag, slot_n(i));
    };
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      half8 a = ring[i % AHEAD];
      if (i + AHEAD < NM) ring[i % AHEAD] = operand(i + AHEAD);
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(reads_after(i)));
      const int n = slot_n(i);
      if (slot_is_u(i)) {
        const int st = n / T::DBLK, b = n % T::DBLK;
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[st], oacc[b], 0, 0, 0);
        if (b == T::DBLK - 1) row_sum(st);
      } else {
        const int kb = n % T::KB, st = n / T::KB;
        const floatx16 c = st == 0 ? floatx16{} : sacc[kb];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[st], c, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- ping-pong schedule -------------------------------------------------------
  // Every wave runs the same sequence of barrier-separated local intervals.
  // 2j is the matrix-core interval of iteration j: U_{j-1} and T_j. 2j+1 is
  // the vector interval: the DMAs of K_{j+3} and V_{j+2}, C_j (mask, exp2,
  // fp16 pack, row max, and when needed the lazy rescale), then the first
  // operands of the next matrix-core interval. Group 1 starts one interval late (an extra barrier up
  // front, which group 0 matches at the end), so in every interval one wave
  // of each SIMD feeds the matrix core while the other runs the vector work.
  // Global interval = local interval + group.
  //
  // Rings (slot = tile % 4). K_t is issued in local 2t-5 and waited for at
  // the end of local 2t-4; after the barrier ending global 2t-3 every wave's
  // share has landed, and it is read from global 2t-1 (group 0's lead
  // operands) to 2t+1. V_t is issued in local 2t-3 and waited for at the end
  // of local 2t-2; visible after global 2t-1, it is read from global 2t+1 to
  // 2t+3. Each wait is vmcnt(0): a vector interval issues K_{j+3} and
  // V_{j+2}, and nothing more before the end of the next matrix-core
  // interval. The next DMA into a K slot (tile t+4) is issued in global 2t+3
  // or later, into a V slot in global 2t+5 or later. The prologue's five
  // DMAs go out whatever the sequence length (past its end they land zeros
  // in slots that are never read); later intervals issue only tiles below
  // n_kv. The last interval, j = n_kv, comes after every wave's last T stage
  // (group 1's in global 2 n_kv - 1, its lead-operand reads in global 2 n_kv),
  // so the K ring is idle from then on: there each wave sends its share of
  // the next tile's Q there.
  auto sync = [&]() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
  auto mfma_sync = [&]() __attribute__((always_inline)) {
    // this wave's K_{j+2} and V_{j+1} DMAs landed
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto vector_sync = [&]() __attribute__((always_inline)) {
    // this wave's operand reads for the next interval are done
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // With Q staging no DMA goes past the key sequence: a zero fill still in
  // flight into the K ring could land on the staged Q.
  auto produce = [&](int j) __attribute__((always_inline)) {
    if (!STAGE_Q || j + 3 < n_kv) fetch_k(j + 3);
    if (!STAGE_Q || j + 2 < n_kv) fetch_v(j + 2);
  };
  // The next tile's Q rows, this wave's share, into the K ring (k-step s of
  // lane l at q_stage + 1024 s + 16 l). Without a next tile the loads read
  // past the buffer (zeros), so that every tile issues the same count.
  auto fetch_q_next = [&]() __attribute__((always_inline)) {
    const int tn = t_next < 0 ? t : t_next;
    const int bh_n = tn / p.n_qt;
    int qt_n = tn - bh_n * p.n_qt;
    if (CAUSAL) qt_n = p.n_qt - 1 - qt_n;
    const __amdgpu_buffer_rsrc_t rq_n = make_rsrc(p.q + (size_t)bh_n * (size_t)N * D, head_bytes);
    const int off = t_next < 0 ? 0x7ffffff0 - 32 * T::KSTEPS
                               : ((qt_n * T::BM + wave * T::QW + l32) * D + 8 * hh) * 2;
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s)
      load16_to_lds(rq_n, off + 32 * s, k_ring + wave * T::KSTEPS * 1024 + 1024 * s);
  };

  // Steady-state iteration j (1 <= j < n_wave) with K slot U = j % 4 known
  // at compile time (V slot (U + 3) % 4), so every LDS operand address is a
  // lane register plus an immediate.
  auto steady = [&](int j, auto u_tag, auto exact_tag) __attribute__((always_inline)) {
    constexpr int U = decltype(u_tag)::value;
    // local interval 2j: matrix core
    __builtin_amdgcn_s_setprio(1);
    mfma_interval(u_tag, std::integral_constant<int, (U + 3) % 4>{});
    __builtin_amdgcn_s_setprio(0);
    mfma_sync();
    // local interval 2j+1: vector ALU
    produce(j);
    if constexpr (decltype(exact_tag)::value) softmax(j);
    else softmax_fast(j);
    prefetch_lead(u_tag);
    vector_sync();
  };
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;
  using U3 = std::integral_constant<int, 3>;
  static_assert(T::SLOTS == 4, "the unrolled loop walks four-slot rings");
  // U stage of a wave's last key tile j - 1 (V slot (j - 1) % 4)
  auto last_pv = [&](int j) __attribute__((always_inline)) {
    switch ((j - 1) & 3) {
      case 0: pv(U0{}); break;
      case 1: pv(U1{}); break;
      case 2: pv(U2{}); break;
      default: pv(U3{}); break;
    }
  };

  // The whole K/V pipeline; the fast variant skips the row max after tile 0.
  auto run_pipeline = [&](auto exact_tag) __attribute__((always_inline)) {
    fetch_k(0);
    fetch_v(0);
    fetch_k(1);
    fetch_k(2);
    fetch_v(1);
    // K_0, V_0 and K_1 landed in every wave (K_2 and V_1 may be in flight)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * T::LOADS_PER_WAVE) : "memory");
    if (group == 1) sync();

    // j = 0: T_0, then C_0
    if (n_wave > 0) qk();
    mfma_sync();
    produce(0);
    if (n_wave > 0) softmax(0);
    prefetch_lead(U0{});
    vector_sync();
    // 1 <= j < n_wave: U_{j-1}, T_j, then C_j
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
    // which the wave still produces its share of the workgroup's tiles
    for (; j <= n_kv; ++j) {
      if (j == n_wave && j >= 1) last_pv(j);
      mfma_sync();
      produce(j);
      if (STAGE_Q && j == n_kv) fetch_q_next();
      vector_sync();
    }
    if (group == 0) sync();
    // Every wave's DMAs but the staged Q loads have landed once all waves
    // pass this barrier: the epilogue and the rerun check reuse the V ring
    // (and without staging the K ring too), across the waves' shares.
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(STAGE_Q ? T::KSTEPS : 0) : "memory");
  };
  // The causal kernel holds the exact pass only: with the fast pass and its
  // rerun compiled in as well, it ran 10% slower on a causal workload with
  // sharp softmax rows (K scaled by 3) and 2% faster on one with plain N(0,1)
  // keys. The fast pass itself is the cheaper one there too; what costs is
  // the reruns' own work. They fall on the heavy causal tiles (up to N / 64
  // key tiles), which have the most chances of a late score far above their
  // first key tile's max; handing tiles out dynamically, so that a rerun only
  // means fewer later tiles, still left the fast pass 2% behind there.
  if constexpr (CAUSAL) {
    run_pipeline(std::true_type{});
  } else {
    run_pipeline(std::false_type{});
    // Any weight overflow shows as a non-finite row sum; the workgroup then
    // reruns with the row max and lazy rescale (the rings are idle here).
    const float l_fast = sum_halves(lacc[0]);
    const bool bad = __builtin_amdgcn_ballot_w64(!(l_fast < INFINITY)) != 0;
    // the flags sit in the V ring (no DMA is in flight any more)
    __attribute__((address_space(3))) int* flags = (__attribute__((address_space(3))) int*)v_ring;
    if (lane == 0) flags[wave] = bad ? 1 : 0;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    int any = 0;
#pragma unroll
    for (int w = 0; w < T::WAVES; ++w) any |= flags[w];
    any = __builtin_amdgcn_readfirstlane(any);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (any) {
      // the next tile's Q is still landing in the K ring, which the rerun
      // refills (it stages that Q again at its end)
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int b = 0; b < T::DBLK; ++b) oacc[b] = floatx16{};
      lacc = floatx4{};
      m_run = -INFINITY;
      run_pipeline(std::true_type{});
    }
  }

  // ---- epilogue: O = O_acc / l, lse = (m + log2 l) * ln 2 -------------------
  // lanes q and q + 32 hold query q; the row sum sits in lane q (lane q + 32 has 0)
  const float l_tot = sum_halves(lacc[0]);
  const float inv = 1.f / l_tot;
  // O goes through LDS (the V ring and the padding after it are idle now;
  // the K ring holds the next tile's Q) so that the global stores are whole
  // rows: each wave writes its 32 rows of fp16 O into a region of its own,
  // rows padded by 16 bytes (a 32-lane write of one d column then hits each
  // bank at most twice, and the 16-byte row reads stay aligned and
  // conflict-free), and stores 16 bytes per lane, D / 8 lanes per row.
  constexpr int O_STRIDE = T::O_STRIDE;
  lds_char* const ob = v_ring + wave * T::QW * O_STRIDE;
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // register 4g + e of block b is d = 32b + 8g + 4hh + e
      half4 w = {(_Float16)(oacc[b][4 * g + 0] * inv), (_Float16)(oacc[b][4 * g + 1] * inv),
                 (_Float16)(oacc[b][4 * g + 2] * inv), (_Float16)(oacc[b][4 * g + 3] * inv)};
      *(__attribute__((address_space(3))) half4*)(ob + l32 * O_STRIDE + (32 * b + 8 * g + 4 * hh) * 2) = w;
    }
  constexpr int LANES_PER_ROW = D / 8;
  constexpr int ROWS_PER_STORE = 64 / LANES_PER_ROW;
  const int srow = lane / LANES_PER_ROW, scol = 8 * (lane % LANES_PER_ROW);
  // Raw-buffer stores, rows at or past N out of range (dropped): every wave
  // issues exactly EPI_STORES of them, which the next tile's wait counts on.
  static_assert(T::QW / ROWS_PER_STORE + 1 == T::EPI_STORES, "epilogue store count");
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + head, head_bytes);
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
  // the next tile's DMAs may refill the rings only once every wave has read
  // its staged rows back
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Persistent schedule (Tawa, sections IV-B and V-E: launch as many
// workgroups as the chip holds and let them iterate over tiles), shared by
// the FP16 and FP8 forward kernels. Workgroup b runs on
// XCD b % 8; the grid is either every tile (one each) or a multiple of 8 no
// larger than the CU count. Pass r hands out slots r * grid .. r * grid +
// grid - 1, walking the workgroups of each XCD in reverse on odd passes, so
// that a workgroup that drew a heavy causal tile draws a light one next.
// Slots map to tile ids so that one XCD's tiles are consecutive ids (one
// head's tiles share its L2). Returns -1 once this workgroup has no tile in
// pass r. With one workgroup per tile there is only pass 0: the reversed
// walk is a permutation of a pass only when the grid is a multiple of 8.
__device__ __forceinline__ int persistent_tile(int r, int G) {
  const int grid = gridDim.x;
  if (r * grid >= G) return -1;
  const int g8 = grid >> 3, b8 = blockIdx.x >> 3, x = blockIdx.x & 7;
  const int slot = r * grid + 8 * ((r & 1) ? g8 - 1 - b8 : b8) + x;
  if (slot >= G) return -1;
  const int per = G >> 3, rem = G & 7;
  return x * per + min(x, rem) + (slot >> 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(Tile<D>::THREADS, 1) void fmha_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Tile<D>::LDS_BYTES];
  const int G = p.total_wg;
  auto tile_of = [&](int r) { return persistent_tile(r, G); };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int r = 0;; ++r) {
    const int t = tile_of(r);
    if (t < 0) break;
    // a non-causal tile stages the next one's Q (see fwd_tile)
    fwd_tile<D, CAUSAL>(p, t, tile_of(r + 1), r > 0, wave, smem_raw);
  }
  // a non-causal workgroup's last tile staged Q loads past the buffer
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace fmha
