// Backward pass of fused multi-head attention for gfx950 (MI355X, CDNA4).
//
// Given Q, K, V, the forward output O, its gradient dO and the forward
// logsumexp, the gradients of sum(dO * O) are, per head,
//   P_ij  = exp(scale * q_i . k_j - lse_i)      (recomputed, never stored)
//   D_i   = dO_i . O_i
//   dS_ij = P_ij * (dO_i . v_j - D_i)
//   dQ    = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO.
// Twill (OSDI'26), sections 6.3 and 6.4, schedules this kernel on Hopper and
// Blackwell: on Hopper it is register-bound and gets no cross-iteration
// pipelining, and FlashAttention 3 uses 80 x 128 tiles there.
//
// Three kernels, each one workgroup per (batch, head, 128-row tile):
// 1. fmha_bwd_delta_kernel: D_i and -lse_i * log2(e) into the workspace
//    (HBM-bound: reads O and dO once).
// 2. fmha_bwd_dkdv_kernel: a workgroup owns 128 keys (32 per wave) and
//    streams every query tile that sees them: S = Q K^T and dP = dO V^T
//    (fp16 MFMA, fp32 accumulate), P and dS on the vector ALU, then
//    dV^T += dO^T P and dK^T += Q^T dS on the matrix core.
// 3. fmha_bwd_dq_kernel: a workgroup owns 128 queries and streams every key
//    tile they see: S^T = K Q^T, dP^T = V dO^T, then dQ^T += K^T dS^T.
// dQ is recomputed in its own pass rather than accumulated with atomics, so
// no workspace beyond D and lse is needed and results are deterministic; the
// price is S and dP computed twice (7 matrix products instead of 5).
//
// Streamed tiles arrive by LDS-DMA (16 bytes per lane straight into LDS, no
// register staging) as [row][d] with 16-byte chunk c of row r at chunk
// c ^ swz(r): in four-slot rings two steps ahead in the dK/dV kernel, in a
// two-slot ring one step ahead in the dQ kernel. One layout serves both
// reads: MFMA A operands of whole rows (ds_read_b128) and transposed A
// operands (ds_read_b64_tr_b16, 8 rows of one d column), both free of LDS
// bank conflicts.
#pragma once

#include "fmha_fwd_kernel.hpp"

namespace fmha {

struct BwdParams {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  const _Float16* o;
  const _Float16* dout;
  const float* lse;
  _Float16* dq;
  _Float16* dk;
  _Float16* dv;
  float* ws;         // [2][rows]: D_i, then -lse_i * log2(e)
  int N;             // sequence length
  int rows;          // B * H * N
  int n_t;           // 128-row tiles per head
  int total_wg;      // B * H * n_t
  float scale_log2;  // scale * log2(e) (any sign: masks apply after scaling)
  float scale;
};

// Sizes shared by the two streaming kernels.
template <int D>
struct BwdTile {
  static constexpr int BT = 128;            // rows (keys or queries) a workgroup owns
  static constexpr int KSTEPS = D / 16;     // MFMA k-steps over d
  static constexpr int DBLK = D / 32;       // 32-row blocks of d
};

// Chunk swizzle of the streamed tiles. For D = 128 (256-byte rows) it is a
// bijection on r mod 16 whose top two bits are r mod 4; for D = 64 (128-byte
// rows) a bijection on (r / 2) mod 8 whose top bit is (r / 2) mod 2. Either
// way 16 consecutive rows read at one chunk, and 4 consecutive rows read at 4
// consecutive chunks, hit distinct banks.
template <int D>
__device__ __forceinline__ int bwd_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int bwd_off(int row, int col) {  // byte offset of element (row, col)
  return row * D * 2 + 16 * ((col >> 3) ^ bwd_swz<D>(row)) + 2 * (col & 7);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . O_i and -lse_i * log2(e)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fmha_bwd_delta_kernel(BwdParams p) {
  constexpr int TPR = D / 8;         // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;     // rows per block
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < p.rows) {
    const half8 a = *reinterpret_cast<const half8*>(p.dout + (size_t)row * D + 8 * c);
    const half8 b = *reinterpret_cast<const half8*>(p.o + (size_t)row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < p.rows && c == 0) {
    p.ws[row] = acc;
    p.ws[p.rows + row] = -p.lse[row] * 1.4426950408889634f;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two streaming kernels
// ---------------------------------------------------------------------------
// Per-lane byte offsets into a streamed [BS][D] tile.
// nat[s]: A operand of row key_of_row(l32) (MFMA row l32), d = 16 s + 8 hh .. +7.
// tr[b][rd]: source of ds_read_b64_tr_b16 for the transposed A operand of
//   d block b, k-step 0, rows 8 hh + 4 rd .. +3 (k-step 1 adds 16 rows). A
//   source lane s of 16-lane group g reads 4 d values starting at column
//   32 b + 16 (g % 2) + 4 sigma(s % 4) of row 8 hh + 4 rd + s / 4, with sigma
//   swapping 1 and 2; result lane i then holds d column
//   32 b + key_of_row(lane % 32), so the accumulator rows come out in
//   natural d order (the same bit-2/3 trick as the row operands).
template <int D>
struct Offsets {
  using T = BwdTile<D>;
  int nat[T::KSTEPS];
  int tr[T::DBLK][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
    const int row = key_of_row(l32);
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s) nat[s] = bwd_off<D>(row, 16 * s + 8 * hh);
    const int s16 = lane & 15, g = lane >> 4;
    const int sig = ((s16 & 1) << 1) | ((s16 >> 1) & 1);
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
        tr[b][rd] = bwd_off<D>(8 * hh + 4 * rd + (s16 >> 2), 32 * b + 16 * (g & 1) + 4 * sig);
  }
};

// XCD-aware tile id: consecutive ids (the tiles of one head) run on one XCD.
__device__ __forceinline__ int bwd_tile_id(int G) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int per = G >> 3, rem = G & 7;
  return xcd * per + min(xcd, rem) + (bid >> 3);
}

// ---------------------------------------------------------------------------
// 2. dK and dV: a workgroup owns 128 keys and streams the query tiles.
// ---------------------------------------------------------------------------
// Eight waves; waves w and w + 4 sit on one SIMD and share the 32 keys
// k0 + 32 (w % 4). Wave w (the P wave) holds K and forms S = Q K^T, P and
// dV^T += dO^T P; wave w + 4 (the dS wave) holds V and forms dP = dO V^T,
// dS = P (dP - D) and dK^T += Q^T dS, taking P from the P wave through LDS.
// Each step (64 queries) has two barrier-separated intervals in which one
// wave of each SIMD feeds the matrix core while the other runs vector work:
//   interval A_t: P wave  MFMA  dV_{t-1}, S_t     | dS wave VALU dS_{t-1}
//   interval B_t: P wave  VALU  P_t (to LDS)      | dS wave MFMA dK_{t-1}, dP_t
// The Q and dO tiles of a step and its two per-query statistics arrive by
// LDS-DMA (no register staging) in four-slot rings, two steps ahead: the
// tiles of step t + 2 are requested during step t and waited for (vmcnt) at
// the end of step t + 1. A wave reads the first operands of its next
// matrix-core interval at the end of its vector interval, so the matrix core
// starts as soon as the barrier opens.
template <int D>
struct DkdvTile {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int PAIRS = 4;
  static constexpr int RW = 32;                  // keys per wave pair
  static constexpr int BT = PAIRS * RW;          // keys per workgroup
  static constexpr int BS = 64;                  // queries per step
  static constexpr int QB = BS / 32;             // 32-query blocks per step
  static constexpr int QSTEPS = BS / 16;         // MFMA k-steps over a step's queries
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int CPR = D / 8;
  static constexpr int TILE_BYTES = BS * D * 2;
  static constexpr int SLOTS = 4;
  static constexpr int RING_BYTES = SLOTS * TILE_BYTES;
  static constexpr int Q_RING = 0;               // Q tiles, one per slot
  static constexpr int DO_RING = RING_BYTES;     // dO tiles
  static constexpr int STAT_BYTES = 2 * BS * 4;  // per slot: D, then -lse * log2(e)
  static constexpr int STATS = 2 * RING_BYTES;
  static constexpr int P_BYTES = QSTEPS * 1024;  // one pair's P (64 x 32 fp16)
  static constexpr int PBUF = STATS + SLOTS * STAT_BYTES;
  static constexpr int LDS_BYTES = PBUF + PAIRS * P_BYTES;
  static constexpr int LOADS_PER_TILE = TILE_BYTES / 1024;  // wave-wide 16-byte-per-lane DMAs
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TILE / WAVES;
  // DMAs a wave issues per step: its share of both tiles and one statistic
  static constexpr int DMA_PER_STEP = 2 * LOADS_PER_WAVE + 1;
  static_assert(LOADS_PER_WAVE >= 1 && LOADS_PER_WAVE * WAVES == LOADS_PER_TILE, "tile DMAs split over the waves");
  static_assert(BS == 64, "one wave-wide 4-byte DMA carries a step's statistic");
  static_assert(RING_BYTES <= 65536, "ring offsets fit a DS instruction's immediate");
  static_assert(DMA_PER_STEP <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "fits the CU's LDS");
};

// LDS reads of the streaming loops are inline asm with explicit lgkmcnt
// waits: as builtins, the compiler cannot tell that they miss the slots an
// LDS-DMA is filling, and would wait for every DMA in flight before each.
// Four 16-byte reads at a + O0 .. a + O3, waited for in the same block.
template <int O0, int O1, int O2, int O3, typename V>
__device__ __forceinline__ void lds_read4_wait(uint32_t a, V (&v)[4]) {
  static_assert(sizeof(V) == 16, "16-byte reads");
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a), "n"(O0), "n"(O1), "n"(O2), "n"(O3)
      : "memory");
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DkdvTile<D>::THREADS, 1) void fmha_bwd_dkdv_kernel(BwdParams p) {
  using T = DkdvTile<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) intx4 lds_intx4;
  __shared__ __attribute__((aligned(16))) char smem_raw[T::LDS_BYTES];
  lds_char* const smem = (lds_char*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool p_wave = wave < 4;
  const int l32 = lane & 31, hh = lane >> 5;

  const int t = bwd_tile_id(p.total_wg);
  const int bh = t / p.n_t;
  const int kt = t - bh * p.n_t;  // causal: low key tiles see the most queries, so go first
  const int N = p.N;
  const int k0 = kt * T::BT;
  const int kw0 = k0 + pair * T::RW;
  const int key = kw0 + l32;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + head, head_bytes);
  // P waves bring each step's -lse * log2(e), dS waves its D (all four waves
  // of a role write the same values)
  const __amdgpu_buffer_rsrc_t rstat =
      make_rsrc(p.ws + (p_wave ? (size_t)p.rows : 0) + (size_t)bh * N, (uint32_t)N * 4u);
  const int stat_which = p_wave ? 1 : 0;

  // This wave's B operand rows: K (P wave) or V (dS wave) of its keys, lane
  // column = key, lane half hh holding d = 16 s + 8 hh .. +7.
  half8 bf[T::KSTEPS];
  {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc((p_wave ? p.k : p.v) + head, head_bytes);
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s)
      bf[s] = __builtin_bit_cast(half8, load16(rb, (key * D + 16 * s + 8 * hh) * 2));
  }
  floatx16 acc[T::DBLK];  // dV^T (P wave) or dK^T (dS wave): lane = key, rows = d
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  const float c2 = p.scale_log2;

  const int q_begin = CAUSAL ? k0 : 0;
  const int n_steps = (N - q_begin + T::BS - 1) / T::BS;

  // ---- producer: step s into ring slot s % 4 --------------------------------
  // Load i of a tile fills LDS chunks 64 i .. 64 i + 63, one per lane; chunk
  // x = row * CPR + pos holds global chunk pos ^ swz(row) of that row (the
  // swizzle is an involution on chunk indices). Steps past the last one read
  // past the end of the head and land zeros; every wave issues exactly
  // DMA_PER_STEP DMAs per step, so the vmcnt counts are fixed.
  int src[T::LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
    const int x = 64 * (wave * T::LOADS_PER_WAVE + i) + lane;
    const int row = x / T::CPR, pos = x % T::CPR;
    src[i] = (row * D + 8 * (pos ^ bwd_swz<D>(row))) * 2;
  }
  auto fetch = [&](int step, auto slot_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    const int q_s = q_begin + step * T::BS;
    const int wofs = wave * T::LOADS_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
      load16_to_lds(rq, q_s * D * 2 + src[i], smem + T::Q_RING + S * T::TILE_BYTES + wofs + i * 1024);
      load16_to_lds(rdo, q_s * D * 2 + src[i], smem + T::DO_RING + S * T::TILE_BYTES + wofs + i * 1024);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rstat, smem + T::STATS + S * T::STAT_BYTES + stat_which * T::BS * 4,
                                             4, (q_s + lane) * 4, 0, 0, 0);
  };

  // ---- consumer-side LDS addresses (per lane; slot and block are immediates)
  // The P wave reads Q as whole rows and dO transposed; the dS wave Q
  // transposed and dO as whole rows.
  Offsets<D> off;
  off.init(lane);
  const uint32_t nat_ring = sbase + (p_wave ? T::Q_RING : T::DO_RING);
  const uint32_t tr_ring = sbase + (p_wave ? T::DO_RING : T::Q_RING);
  uint32_t nat_rd[T::KSTEPS], tr_rd[T::DBLK][2];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s) nat_rd[s] = nat_ring + off.nat[s];
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) tr_rd[b][rd] = tr_ring + off.tr[b][rd];
  // statistics: query 32 qb + 16 (i / 8) + 8 hh + i % 8 of the step for
  // accumulator register i; P of a pair: 1024 bytes per 16-query k-step
  const uint32_t stat_rd = sbase + T::STATS + 4 * 8 * hh;
  const uint32_t p_rw = sbase + T::PBUF + pair * T::P_BYTES + 16 * lane;

  // S (P wave) or dP (dS wave) of the newest step, per 32-query block: lane
  // = key, register i = query 32 qb + 16 (i / 8) + 8 hh + i % 8 of the step
  floatx16 sc[T::QB];
  // P (P wave) or dS (dS wave) of the previous step in fp16, per 16-query
  // k-step: w16[2 qb + i / 8][i % 8] is register i of block qb
  half8 w16[T::QSTEPS];

  // Matrix-core interval: acc += (transposed tile of step t-1)^T w16 (NC =
  // DBLK x QSTEPS MFMAs), then sc = (row tile of step t) bf (QB x KSTEPS),
  // in a fixed order in which consecutive MFMAs of one kind alternate
  // accumulators. Operand i is read AHEAD MFMAs before its use (the first
  // AHEAD by `prefetch`, before the interval's barrier), and MFMA i waits
  // only for its own operand: LDS reads complete in order. It always runs
  // whole: w16 is zero when step t-1 contributes nothing (the ring's
  // previous slot holds finite values), and sc is unused when step t is
  // inactive.
  constexpr int NC = T::DBLK * T::QSTEPS, NM = NC + T::QB * T::KSTEPS, AHEAD = OPERAND_AHEAD;
  static_assert(AHEAD <= NC, "the prefetched operands are all from the previous step's tile");
  auto reads_of = [](int i) constexpr { return i < NC ? 2 : 1; };
  auto reads_after = [reads_of](int i) constexpr {
    int r = 0;
    for (int m = i + 1; m < i + AHEAD && m < NM; ++m) r += reads_of(m);
    return r;
  };
  static_assert(reads_after(0) <= 15 && reads_after(NC - AHEAD) <= 15, "lgkmcnt range");
  auto operand = [&](auto ps_tag, auto cs_tag, int i) __attribute__((always_inline)) {
    constexpr int PS = decltype(ps_tag)::value, CS = decltype(cs_tag)::value;
    half8 a;
    if (i < NC) {
      const int b = i % T::DBLK, ks = i / T::DBLK;
      shortx4 lo, hi;
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(lo)
                   : "v"(tr_rd[b][0]), "i"(PS * T::TILE_BYTES + ks * 16 * D * 2));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(hi)
                   : "v"(tr_rd[b][1]), "i"(PS * T::TILE_BYTES + ks * 16 * D * 2));
      a = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      const int n = i - NC, qb = n % T::QB, k = n / T::QB;
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(a)
                   : "v"(nat_rd[k]), "i"(CS * T::TILE_BYTES + qb * 32 * D * 2));
    }
    return a;
  };
  half8 ring[AHEAD];
  auto prefetch = [&](auto ps_tag) __attribute__((always_inline)) {
    using C0 = std::integral_constant<int, 0>;
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ring[i] = operand(ps_tag, C0{}, i);
  };
  auto mfma_interval = [&](auto ps_tag, auto cs_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      half8 a = ring[i % AHEAD];
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(reads_after(i)));
      if (i + AHEAD < NM) ring[i % AHEAD] = operand(ps_tag, cs_tag, i + AHEAD);
      if (i < NC) {
        const int b = i % T::DBLK, ks = i / T::DBLK;
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w16[ks], acc[b], 0, 0, 0);
      } else {
        const int n = i - NC, qb = n % T::QB, k = n / T::QB;
        const floatx16 c = k == 0 ? floatx16{} : sc[qb];
        sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bf[k], c, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto zero_w16 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < T::QSTEPS; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) w16[k][i] = (_Float16)0.f;
  };
  // per-query statistic `which` of query block qb, as laid out in the
  // accumulators: v[g][e] for register 4 g + e
  auto stats = [&](auto slot_tag, auto which_tag, auto qb_tag, floatx4 (&v)[4]) __attribute__((always_inline)) {
    constexpr int O = decltype(slot_tag)::value * T::STAT_BYTES + decltype(which_tag)::value * T::BS * 4 +
                      decltype(qb_tag)::value * 32 * 4;
    lds_read4_wait<O, O + 16, O + 64, O + 80>(stat_rd, v);
  };

  // a causal step entirely before the pair's first key contributes nothing
  auto active = [&](int step) __attribute__((always_inline)) {
    return step >= 0 && step < n_steps && (!CAUSAL || q_begin + step * T::BS + T::BS - 1 >= kw0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // One step t in the role of this wave; U = t mod 4 is compile-time, so
  // every LDS address is a lane register plus an immediate.
  auto p_step = [&](int t, auto u_tag) __attribute__((always_inline)) {
    constexpr int U = decltype(u_tag)::value;
    using PREV = std::integral_constant<int, (U + 3) % 4>;
    using CUR = std::integral_constant<int, U>;
    using FILL = std::integral_constant<int, (U + 2) % 4>;
    // interval A: dV^T += dO^T P (step t-1), then S = Q K^T (step t)
    __builtin_amdgcn_s_setprio(1);
    mfma_interval(PREV{}, CUR{});
    __builtin_amdgcn_s_setprio(0);
    asm volatile("s_barrier" ::: "memory");
    // interval B: P = 2^(S c - lse log2 e) in fp16, to registers and LDS
    if (active(t)) {
      const int q_s = q_begin + t * T::BS;
      // base-2 exponents s c - lse log2 e (any finite scale)
      {
        floatx4 nl[4];
        stats(CUR{}, I1{}, I0{}, nl);
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[0][i] = __builtin_fmaf(sc[0][i], c2, nl[i >> 2][i & 3]);
        stats(CUR{}, I1{}, I1{}, nl);
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[1][i] = __builtin_fmaf(sc[1][i], c2, nl[i >> 2][i & 3]);
      }
      // Masked exponents become -inf (weight 0), on edge steps only: the test
      // is uniform, so other steps branch past it.
      const bool edge = (CAUSAL && q_s < kw0 + T::RW - 1) || q_s + T::BS > N || kw0 + T::RW > N;
      if (edge) {
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = q_s + 32 * qb + 16 * (i >> 3) + 8 * hh + (i & 7);
            if ((CAUSAL && q < key) || q >= N || key >= N) sc[qb][i] = -INFINITY;
          }
      }
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          w16[2 * qb + (i >> 3)][i & 7] = (_Float16)__builtin_amdgcn_exp2f(sc[qb][i]);
      static_assert(T::QSTEPS == 4, "four 16-byte P writes per lane");
      asm volatile(
          "ds_write_b128 %0, %1\n\t"
          "ds_write_b128 %0, %2 offset:1024\n\t"
          "ds_write_b128 %0, %3 offset:2048\n\t"
          "ds_write_b128 %0, %4 offset:3072"
          :
          : "v"(p_rw), "v"(w16[0]), "v"(w16[1]), "v"(w16[2]), "v"(w16[3])
          : "memory");
    } else {
      zero_w16();
    }
    fetch(t + 2, FILL{});
    // the next interval's first operands: dO of this step, transposed
    if (t < n_steps) prefetch(CUR{});
    // end of step: step t + 1's tiles have landed (only step t + 2's DMAs
    // may be pending) and the P writes are done (issued before the
    // prefetch's 2 AHEAD reads)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(%1)\n\ts_barrier" ::"n"(T::DMA_PER_STEP), "n"(2 * AHEAD) : "memory");
  };
  auto ds_step = [&](int t, auto u_tag) __attribute__((always_inline)) {
    constexpr int U = decltype(u_tag)::value;
    using PREV = std::integral_constant<int, (U + 3) % 4>;
    using CUR = std::integral_constant<int, U>;
    using FILL = std::integral_constant<int, (U + 2) % 4>;
    fetch(t + 2, FILL{});
    // interval A: dS = P (dP - D) of step t-1, P from the P wave
    if (active(t - 1)) {
      half8 pw[4];
      lds_read4_wait<0, 1024, 2048, 3072>(p_rw, pw);
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) {
        floatx4 dd[4];
        if (qb == 0) stats(PREV{}, I0{}, I0{}, dd);
        else stats(PREV{}, I0{}, I1{}, dd);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = (float)pw[2 * qb + (i >> 3)][i & 7];
          w16[2 * qb + (i >> 3)][i & 7] = (_Float16)(pv * (sc[qb][i] - dd[i >> 2][i & 3]));
        }
      }
    } else {
      zero_w16();
    }
    // interval B's first operands: Q of step t-1, transposed
    prefetch(PREV{});
    asm volatile("s_barrier" ::: "memory");
    // interval B: dK^T += Q^T dS (step t-1), then dP = dO V^T (step t)
    __builtin_amdgcn_s_setprio(1);
    mfma_interval(PREV{}, CUR{});
    __builtin_amdgcn_s_setprio(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(T::DMA_PER_STEP) : "memory");
  };
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;
  using U3 = std::integral_constant<int, 3>;

  // prologue: slot 3 (step 0's "previous" slot) zeroed, steps 0 and 1
  // requested, step 0 waited for
  for (int x = tid; x < T::TILE_BYTES / 16; x += T::THREADS) {
    *(lds_intx4*)(smem + T::Q_RING + 3 * T::TILE_BYTES + 16 * x) = intx4{0, 0, 0, 0};
    *(lds_intx4*)(smem + T::DO_RING + 3 * T::TILE_BYTES + 16 * x) = intx4{0, 0, 0, 0};
  }
  fetch(0, U0{});
  fetch(1, U1{});
  zero_w16();
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(T::DMA_PER_STEP) : "memory");
  // bf (loaded before the DMAs) has landed too; passing it through an empty
  // asm tells the compiler so, which keeps it from waiting for every DMA in
  // flight before the loop
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s) asm volatile("" : "+v"(bf[s]));
  // steps 0 .. n_steps (the last one only finishes step n_steps - 1)
  if (p_wave) {
    prefetch(U3{});
    int t = 0;
    for (; t + 3 <= n_steps; t += 4) {
      p_step(t, U0{});
      p_step(t + 1, U1{});
      p_step(t + 2, U2{});
      p_step(t + 3, U3{});
    }
    if (t <= n_steps) p_step(t, U0{});
    if (t + 1 <= n_steps) p_step(t + 1, U1{});
    if (t + 2 <= n_steps) p_step(t + 2, U2{});
  } else {
    int t = 0;
    for (; t + 3 <= n_steps; t += 4) {
      ds_step(t, U0{});
      ds_step(t + 1, U1{});
      ds_step(t + 2, U2{});
      ds_step(t + 3, U3{});
    }
    if (t <= n_steps) ds_step(t, U0{});
    if (t + 1 <= n_steps) ds_step(t + 1, U1{});
    if (t + 2 <= n_steps) ds_step(t + 2, U2{});
  }
  // the DMAs of the two steps past the end must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  // epilogue: register i of block b holds d = 32 b + 16 (i / 8) + 8 hh + i % 8
  if (key < N) {
    _Float16* dst = (p_wave ? p.dv : p.dk) + head + (size_t)key * D;
    const float f = p_wave ? 1.f : p.scale;
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        half8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (_Float16)(acc[b][8 * g + e] * f);
        *reinterpret_cast<half8*>(dst + 32 * b + 16 * g + 8 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: a workgroup owns 128 queries and streams the key tiles.
// ---------------------------------------------------------------------------
// Four waves of 32 queries; two workgroups share a CU. Key and value tiles
// of 64 rows stream by LDS-DMA (16 bytes per lane straight into LDS, no
// register staging) into a two-slot ring; each wave issues a quarter of each
// tile. The step loop is unrolled by two so that both slots are compile-time
// offsets, which keeps the compiler from waiting for the DMA in flight
// before reading the other slot.
template <int D>
struct DqTile {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int RW = 32;               // queries a wave owns
  static constexpr int BT = WAVES * RW;       // queries a workgroup owns
  static constexpr int BS = 64;               // keys per step
  static constexpr int KB = BS / 32;          // 32-key blocks per step
  static constexpr int KSTEPS = D / 16;       // MFMA k-steps over d
  static constexpr int DBLK = D / 32;         // 32-row blocks of dQ^T
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int TILE_BYTES = BS * D * 2;
  static constexpr int SLOT_BYTES = 2 * TILE_BYTES;  // K tile, then V tile
  static constexpr int LDS_BYTES = 2 * SLOT_BYTES;
  static constexpr int LOADS_PER_TILE = TILE_BYTES / 1024;  // wave-wide 16-byte-per-lane loads
  static constexpr int LOADS_PER_WAVE = LOADS_PER_TILE / WAVES;
  static_assert(LOADS_PER_WAVE * WAVES == LOADS_PER_TILE, "tile loads split over the waves");
  static_assert(BT == BwdTile<D>::BT, "the dQ grid tiles 128 queries like the other kernels");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DqTile<D>::THREADS, 2) void fmha_bwd_dq_kernel(BwdParams p) {
  using T = DqTile<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) half8 lds_half8;
  __shared__ __attribute__((aligned(16))) char smem_raw[T::LDS_BYTES];
  lds_char* const smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int t = bwd_tile_id(p.total_wg);
  const int bh = t / p.n_t;
  int qt = t - bh * p.n_t;
  if (CAUSAL) qt = p.n_t - 1 - qt;  // heaviest query tiles first
  const int N = p.N;
  const int q0 = qt * T::BT;
  const int qw0 = q0 + wave * T::RW;
  const int qrow = qw0 + l32;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rD = make_rsrc(p.ws + (size_t)bh * N, (uint32_t)N * 4u);
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(p.ws + p.rows + (size_t)bh * N, (uint32_t)N * 4u);

  // Q and dO rows of this wave's queries: B operands of S^T = K Q^T and
  // dP^T = V dO^T. Per-query statistics are per-lane scalars here.
  half8 qf[T::KSTEPS], dof[T::KSTEPS];
#pragma unroll
  for (int s = 0; s < T::KSTEPS; ++s) {
    qf[s] = __builtin_bit_cast(half8, load16(rq, (qrow * D + 16 * s + 8 * hh) * 2));
    dof[s] = __builtin_bit_cast(half8, load16(rdo, (qrow * D + 16 * s + 8 * hh) * 2));
  }
  const float Dq = load_f32(rD, qrow * 4);
  const float nl2 = load_f32(rL, qrow * 4);
  floatx16 dqt[T::DBLK];  // dQ^T: lane = query, rows = d
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqt[b][i] = 0.f;

  // DMA sources: load L of a tile fills LDS chunks 64 L .. 64 L + 63, one per
  // lane; chunk x = row * CPR + pos holds global chunk pos ^ swz(row) of that
  // row (the swizzle is an involution on chunk indices).
  int src[T::LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
    const int x = 64 * (wave * T::LOADS_PER_WAVE + i) + lane;
    const int row = x / T::CPR, pos = x % T::CPR;
    src[i] = (row * D + 8 * (pos ^ bwd_swz<D>(row))) * 2;
  }
  auto fetch = [&](int step, auto slot_tag) __attribute__((always_inline)) {
    lds_char* dst = smem + decltype(slot_tag)::value * T::SLOT_BYTES + wave * T::LOADS_PER_WAVE * 1024;
    const int base = step * T::BS * D * 2;
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
      load16_to_lds(rk, base + src[i], dst + i * 1024);
      load16_to_lds(rv, base + src[i], dst + T::TILE_BYTES + i * 1024);
    }
  };

  Offsets<D> off;
  off.init(lane);
  const float c2 = p.scale_log2;

  const int k_end = CAUSAL ? min(N, q0 + T::BT) : N;
  const int n_steps = (k_end + T::BS - 1) / T::BS;

  // LDS operand addresses: a lane register plus an immediate (slot, tile,
  // key block or k-step). Row operands of S^T = K Q^T and dP^T = V dO^T
  // (K or V row key_of_row(l32) of the 32-key block, d = 16 k + 8 hh ..),
  // and the transposed K operand of dQ^T += K^T dS^T.
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  uint32_t nat_rd[T::KSTEPS], tr_rd[T::DBLK][2];
#pragma unroll
  for (int k = 0; k < T::KSTEPS; ++k) nat_rd[k] = sbase + off.nat[k];
#pragma unroll
  for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) tr_rd[b][rd] = sbase + off.tr[b][rd];
  // S/dP MFMA i: k-step i / 4, key block (i / 2) % 2, K (even i) or V (odd
  // i); dQ MFMA i: k-step i / DBLK over the step's keys, d block i % DBLK.
  // Consecutive MFMAs never share an accumulator. Each operand is read
  // AHEAD MFMAs before its use and waited for alone (LDS reads complete in
  // order). The reads are inline asm: as builtins the compiler cannot tell
  // that they miss the slot an LDS-DMA is filling, and it waits for every
  // DMA in flight before each.
  constexpr int NSD = 4 * T::KSTEPS, NDQ = 4 * T::DBLK, AHEAD = OPERAND_AHEAD;
  static_assert(T::KB == 2 && NSD >= AHEAD && NDQ >= AHEAD, "interval shapes");
  auto sd_operand = [&](auto slot_tag, int i) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    const int k = i >> 2, kb = (i >> 1) & 1, is_v = i & 1;
    half8 a;
    asm volatile("ds_read_b128 %0, %1 offset:%2"
                 : "=v"(a)
                 : "v"(nat_rd[k]), "i"(SLOT * T::SLOT_BYTES + is_v * T::TILE_BYTES + kb * 32 * D * 2));
    return a;
  };
  auto dq_operand = [&](auto slot_tag, int i) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    const int ks = i / T::DBLK, b = i % T::DBLK;
    shortx4 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(lo)
                 : "v"(tr_rd[b][0]), "i"(SLOT * T::SLOT_BYTES + ks * 16 * D * 2));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(hi)
                 : "v"(tr_rd[b][1]), "i"(SLOT * T::SLOT_BYTES + ks * 16 * D * 2));
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One step: wait until this wave's part of tile `step` has landed, then a
  // barrier (every part has landed, and every wave is done with the other
  // slot); start the next tile's DMA into the other slot; compute.
  auto run_step = [&](int step, auto cur_tag, auto nxt_tag) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (step + 1 < n_steps) fetch(step + 1, nxt_tag);
    const int k_s = step * T::BS;
    if (CAUSAL && k_s > qw0 + T::RW - 1) return;  // every key of the step is after every query
    // S^T = K Q^T and dP^T = V dO^T per 32-key block: lane = query, register
    // i = key k_s + 32 kb + 16 (i / 8) + 8 hh + i % 8.
    floatx16 s[T::KB], dp[T::KB];
    half8 ring[AHEAD];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ring[i] = sd_operand(cur_tag, i);
#pragma unroll
    for (int i = 0; i < NSD; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      half8 a = ring[i % AHEAD];
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(NSD - 1 - i < AHEAD - 1 ? NSD - 1 - i : AHEAD - 1));
      if (i + AHEAD < NSD) ring[i % AHEAD] = sd_operand(cur_tag, i + AHEAD);
      const int k = i >> 2, kb = (i >> 1) & 1;
      if (i & 1) dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, dof[k], k == 0 ? floatx16{} : dp[kb], 0, 0, 0);
      else s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[k], k == 0 ? floatx16{} : s[kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the dQ interval's first operands land during the vector work
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ring[i] = dq_operand(cur_tag, i);
    // base-2 exponents s c - lse log2 e (any finite scale)
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_fmaf(s[kb][i], c2, nl2);
    // Masked exponents become -inf (weight 0), on edge steps only: the test
    // is uniform, so other steps branch past it.
    const bool edge = (CAUSAL && k_s + T::BS - 1 > qw0) || k_s + T::BS > N;
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = k_s + 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
          if ((CAUSAL && kk > qrow) || kk >= N) s[kb][i] = -INFINITY;
        }
    }
    half8 dsf[2 * T::KB];
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(s[kb][i]);
        dsf[2 * kb + (i >> 3)][i & 7] = (_Float16)(pv * (dp[kb][i] - Dq));
      }
    // dQ^T += K^T dS^T (k = keys, 16 per k-step)
    static_assert(2 * T::KB == 4, "four 16-key k-steps per step");
#pragma unroll
    for (int i = 0; i < NDQ; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      half8 a = ring[i % AHEAD];
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(2 * (NDQ - 1 - i < AHEAD - 1 ? NDQ - 1 - i : AHEAD - 1)));
      if (i + AHEAD < NDQ) ring[i % AHEAD] = dq_operand(cur_tag, i + AHEAD);
      const int ks = i / T::DBLK, b = i % T::DBLK;
      dqt[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, dsf[ks], dqt[b], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  if (n_steps > 0) fetch(0, Slot0{});
  for (int step = 0; step < n_steps; step += 2) {
    run_step(step, Slot0{}, Slot1{});
    if (step + 1 < n_steps) run_step(step + 1, Slot1{}, Slot0{});
  }
  // no DMA is in flight past the last step (it issues none)

  if (qrow < N) {
    _Float16* dqr = p.dq + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        half8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (_Float16)(dqt[b][8 * g + e] * p.scale);
        *reinterpret_cast<half8*>(dqr + 32 * b + 16 * g + 8 * hh) = w;
      }
  }
}

}  // namespace fmha
