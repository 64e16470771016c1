// Warp-specialised fp16 GEMM for gfx950 (MI355X, CDNA4): C = A B with A
// [M][K], B [K][N] and C [M][N] row-major binary16, fp32 accumulation.
//
// Structure (performance-model page for warp-specialised kernels, sections
// "Warp specialization kernel structure" and "Algorithm 1"): each workgroup
// computes one T_M x T_N output tile in S = ceil(K / T_K) stages, with two
// kinds of wave.
// - One DMA wave moves each stage's A tile (T_M x T_K) and B tile
//   (T_K x T_N) from HBM into a ring of RING slots in LDS by LDS-DMA
//   (buffer_load ... lds). It waits while the ring is full.
// - Four MATH waves (one per SIMD, each a quarter of the tile) read the
//   stage's operands from LDS into registers, run the fp16 MFMAs, release
//   the slot, and finally store their part of C.
// The page's wait()/signal() semaphores are counters in LDS: `full` (stages
// landed, written by the DMA wave) and one `released` counter per MATH wave
// (stages that wave has finished reading). The DMA wave reuses a slot once
// the slowest MATH wave has released it: MATH waves run independently, so a
// single summed count could be reached while one wave still reads the slot.
// Waiting is polling with s_sleep. Every poll loop
// is bounded, and a wave that gives up reports it through the status word,
// so no wave can wait forever.
//
// The DMA wave keeps up to two stages in flight. A stage has landed once the
// wave's vmcnt shows its loads done (loads complete in issue order; a stage
// of more than 63 loads is settled between the next stage's A and B loads). Before
// it blocks on a full ring it signals everything it has issued, so the MATH
// waves can always drain the ring.
//
// gfx950 mapping. The product is formed transposed, C^T = B^T A^T, with
// v_mfma_f32_32x32x16_f16: the B^T operand (rows n, 8 consecutive k per
// lane) comes from the row-major B tile through ds_read_b64_tr_b16, and the
// A^T operand (8 consecutive k of one row m per lane) is one 16-byte read
// of the row-major A tile. Each accumulator lane then holds one row m and 4
// consecutive columns n per register group, stored as 8-byte writes.
// Both LDS tiles are swizzled in 16-byte chunks so that these reads hit
// distinct banks; the DMA wave writes that layout directly by choosing each
// lane's source address.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsgemm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

struct GemmParams {
  const _Float16* a;
  const _Float16* b;
  _Float16* c;
  unsigned long long* trace;  // optional per-stage timestamps (see below)
  int* status;                // optional; set to 1 if any wait gave up
  int M, N, K;
  int n_tm, n_tn;             // output tiles along M and N
  int stages;                 // ceil(K / T_K)
  int spin_limit;             // polls before a wait gives up
};

// Trace layout, when p.trace is not null: per workgroup (launch order) a
// block of (stages + 1) x 5 values of wall_clock64() (100 MHz). Row i < S:
// [0] DMA wave starts issuing stage i, [1] DMA wave sees stage i landed and
// signals it, [2] MATH wave 0 starts stage i, [3] MATH wave 0 releases
// stage i's slot, [4] MATH wave 0's MFMAs of stage i have finished. Row S:
// [0] workgroup start, [1] MATH wave 0 done with its stores, [2] the tile
// id, [3] and [4] 0. Only a traced launch waits for [4] (a register read of
// the stage's last accumulator), so only it is slowed by it.
constexpr int TRACE_FIELDS = 5;
// One DMA wave and four MATH waves.
constexpr int GEMM_THREADS = 5 * 64;

template <int TM, int TN, int TK, int RING>
struct GemmTile {
  static constexpr int MATH_WAVES = 4;
  static constexpr int THREADS = GEMM_THREADS;
  static constexpr int MB = TM / 64;       // 32-row blocks per MATH wave (a wave has TM/2 rows)
  static constexpr int NB = TN / 64;       // 32-column blocks per MATH wave
  static constexpr int KSTEPS = TK / 16;   // MFMA k-steps per stage
  static constexpr int CA = TK / 8;        // 16-byte chunks per A tile row
  static constexpr int CB = TN / 8;        // 16-byte chunks per B tile row
  static constexpr int A_BYTES = TM * TK * 2;
  static constexpr int B_BYTES = TK * TN * 2;
  static constexpr int SLOT_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024;  // 1 KB per wave-wide LDS-DMA
  static constexpr int B_LOADS = B_BYTES / 1024;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int RING_BYTES = RING * SLOT_BYTES;
  // At least 82 KB, so one workgroup occupies a CU (the model's unit).
  static constexpr int LDS_BYTES = (RING_BYTES + 64 > 82 * 1024) ? RING_BYTES + 64 : 82 * 1024;
  static_assert(TM == 64 || TM == 128 || TM == 256, "T_M");
  static_assert(TN == 64 || TN == 128, "T_N");
  static_assert(TK == 64 || TK == 128, "T_K");
  static_assert(RING >= 1 && RING <= 4, "ring depth");
  static_assert(A_LOADS <= 63 && B_LOADS <= 63, "vmcnt holds 63");
  static_assert(LDS_BYTES <= 160 * 1024, "fits the CU's LDS");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer: loads at or past `bytes` return zeros.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds_base + 16 l (buffer_load_dwordx4 ... lds). lds_base must be uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int byte_off, lds_char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, byte_off, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma16(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Offset that is always out of range (buffers are below 2^31 bytes).
constexpr int OOB = 0x7ffffff0;

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) {
  return (uint32_t)(uintptr_t)p;
}

// Poll an LDS counter until it reaches `target`. Inline asm keeps the
// compiler from waiting on this wave's LDS-DMA before the read. Returns
// false if it gave up after `limit` polls.
__device__ __forceinline__ bool wait_geq(const lds_char* cnt, uint32_t target, int limit) {
  for (int n = 0; n < limit; ++n) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(cnt)) : "memory");
    if (__builtin_amdgcn_readfirstlane(v) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Poll four consecutive LDS counters until their minimum reaches `target`.
__device__ __forceinline__ bool wait_min4_geq(const lds_char* cnt, uint32_t target, int limit) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  for (int n = 0; n < limit; ++n) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(cnt)) : "memory");
    const uint32_t m = min(min(v[0], v[1]), min(v[2], v[3]));
    if (__builtin_amdgcn_readfirstlane(m) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// ds_read_b64_tr_b16: in each 16-lane group, lane i supplies the address of
// 4 consecutive halves of row i/4 of a 4 x 16 block and receives column i
// of its 4 rows. (A device function of its own: the builtin exists only for
// gfx950, and the host pass must still see a valid kernel template.)
__device__ __forceinline__ shortx4 read_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)p);
}

__device__ __forceinline__ void store_counter(lds_char* cnt, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(cnt)), "v"(v) : "memory");
}

template <int TM, int TN, int TK, int RING>
__global__ __launch_bounds__(GEMM_THREADS) void ws_gemm_kernel(GemmParams p) {
  using T = GemmTile<TM, TN, TK, RING>;
  __shared__ __attribute__((aligned(16))) char smem_raw[T::LDS_BYTES];
  lds_char* const ring = (lds_char*)smem_raw;
  lds_char* const full = ring + T::RING_BYTES;   // stages landed
  lds_char* const released = full + 16;         // per MATH wave: stages released

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = p.stages;
  const int limit = p.spin_limit;

  // Tile id: workgroups go round-robin over the 8 XCDs (bid % 8); renumber
  // so that each XCD takes consecutive ids. Ids walk groups of 4 tile rows
  // column by column, so the tiles that run together on one XCD share A
  // and B panels in its L2.
  const int G = p.n_tm * p.n_tn;
  const int bid = blockIdx.x, per = G >> 3, rem = G & 7, x = bid & 7;
  const int t = x * per + (x < rem ? x : rem) + (bid >> 3);
  constexpr int GROUP = 4;
  const int group = t / (GROUP * p.n_tn);
  const int rows_in_group = min(GROUP, p.n_tm - group * GROUP);
  const int in_group = t - group * GROUP * p.n_tn;
  const int tm = group * GROUP + in_group % rows_in_group;
  const int tn = in_group / rows_in_group;
  const int m0 = tm * TM, n0 = tn * TN;

  unsigned long long* const trace = p.trace ? p.trace + (size_t)bid * (S + 1) * TRACE_FIELDS : nullptr;

  if (tid < 1 + T::MATH_WAVES) {
    store_counter(tid == 0 ? full : released + 4 * (tid - 1), 0u);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  __syncthreads();

  if (wave == T::MATH_WAVES) {
    // ---------------- DMA wave ----------------
    if (trace && lane == 0) trace[S * TRACE_FIELDS + 0] = wall_clock64();
    const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(p.a, (uint32_t)p.M * p.K * 2u);
    const __amdgpu_buffer_rsrc_t rb = gemm_rsrc(p.b, (uint32_t)p.K * p.N * 2u);
    // Per load instruction: the global element this lane fetches at k0 = 0,
    // and its column (k for A, n for B) for the bounds test.
    int a_off[T::A_LOADS], a_col[T::A_LOADS];
#pragma unroll
    for (int j = 0; j < T::A_LOADS; ++j) {
      const int xx = 64 * j + lane, r = xx / T::CA, pos = xx % T::CA;
      const int c = pos ^ (r % T::CA);
      a_col[j] = 8 * c;
      a_off[j] = (m0 + r) * p.K + 8 * c;
    }
    int b_off[T::B_LOADS], b_col[T::B_LOADS];
#pragma unroll
    for (int j = 0; j < T::B_LOADS; ++j) {
      const int xx = 64 * j + lane, kr = xx / T::CB, pos = xx % T::CB;
      const int c = pos ^ ((T::CB == 16 ? 4 : 2) * (kr & 3));
      b_col[j] = n0 + 8 * c;
      b_off[j] = kr * p.N + n0 + 8 * c;
    }
    bool ok = true, pending = false;
    for (int i = 0; i < S; ++i) {
      if (i >= RING) {
        const uint32_t need = (uint32_t)(i - RING + 1);  // stage i - RING released by all
        if (pending && !wait_min4_geq(released, need, 1)) {
          // The ring is full: signal what is in flight before blocking, so
          // that the MATH waves can drain it.
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (trace && lane == 0) trace[(i - 1) * TRACE_FIELDS + 1] = wall_clock64();
          if (lane == 0) store_counter(full, (uint32_t)i);
          pending = false;
        }
        ok = ok && wait_min4_geq(released, need, limit);
      }
      if (trace && lane == 0) trace[i * TRACE_FIELDS + 0] = wall_clock64();
      lds_char* const slot = ring + (i % RING) * T::SLOT_BYTES;
      const int k0 = i * TK;
#pragma unroll
      for (int j = 0; j < T::A_LOADS; ++j) {
        const int off = (k0 + a_col[j] < p.K) ? 2 * (a_off[j] + k0) : OOB;
        dma16(ra, off, slot + 1024 * j);
      }
      if constexpr (T::LOADS > 63) {
        // A stage is more loads than vmcnt can count: settle stage i-1
        // between stage i's A and B loads.
        if (pending) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::A_LOADS) : "memory");
          if (trace && lane == 0) trace[(i - 1) * TRACE_FIELDS + 1] = wall_clock64();
          if (lane == 0) store_counter(full, (uint32_t)i);
          pending = false;
        }
      }
#pragma unroll
      for (int j = 0; j < T::B_LOADS; ++j) {
        const int off = (b_col[j] < p.N) ? 2 * (b_off[j] + k0 * p.N) : OOB;
        dma16(rb, off, slot + T::A_BYTES + 1024 * j);
      }
      if constexpr (T::LOADS <= 63) {
        if (pending) {  // all but stage i's loads have landed: stage i-1 is in
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::LOADS) : "memory");
          if (trace && lane == 0) trace[(i - 1) * TRACE_FIELDS + 1] = wall_clock64();
          if (lane == 0) store_counter(full, (uint32_t)i);
        }
      }
      pending = true;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (S > 0) {
      if (trace && lane == 0) trace[(S - 1) * TRACE_FIELDS + 1] = wall_clock64();
      if (lane == 0) store_counter(full, (uint32_t)S);
    }
    if (!ok && p.status && lane == 0) *p.status = 1;
    return;
  }

  // ---------------- MATH waves ----------------
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  // A^T operand: row m = wm*TM/2 + 32*mb + l32 of the A tile, chunk 2*s + hh
  // of k-step s, stored at chunk ^ (row % CA).
  int a_row[T::MB], a_swz[T::MB];
#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb) {
    const int r = wm * (TM / 2) + 32 * mb + l32;
    a_row[mb] = r * TK * 2;
    a_swz[mb] = r % T::CA;
  }
  // B^T operand by ds_read_b64_tr_b16: in 16-lane group g, lane i reads 4
  // columns (col .. col+3) of k-row 8*(g/2) + i/4 (+ 16 s + 4 q), and
  // receives column 16*(g%2) + i of 4 consecutive k-rows.
  int b_base[T::NB];
  {
    const int g = lane >> 4, i = lane & 15;
    const int kr = 8 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
      const int col = wn * (TN / 2) + 32 * nb + 16 * (g & 1) + 4 * (i & 3);
      const int c = (col >> 3) ^ ((T::CB == 16 ? 4 : 2) * (kr & 3));
      b_base[nb] = T::A_BYTES + kr * TN * 2 + 16 * c + 2 * (col & 7);
    }
  }

  floatx16 acc[T::MB][T::NB];
#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // Operands of one k-step: A^T fragments by 16-byte reads, B^T fragments
  // by pairs of transposing reads.
  auto read_step = [&](const lds_char* slot, int s, half8 (&af)[T::MB], half8 (&bf)[T::NB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
      af[mb] = *(const __attribute__((address_space(3))) half8*)(
          slot + a_row[mb] + 16 * ((2 * s + hh) ^ a_swz[mb]));
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
      const lds_char* src = slot + b_base[nb] + 16 * s * TN * 2;
      const shortx4 lo = read_tr16(src);
      const shortx4 hi = read_tr16(src + 4 * TN * 2);
      bf[nb] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  // Software pipeline over k-steps, one step ahead, across stage boundaries:
  // at the last step of stage i the wave completes stage i's reads, releases
  // its slot, waits for stage i+1 and reads its first operands, all before
  // stage i's last MFMAs.
  static_assert(T::KSTEPS % 2 == 0, "k-step buffers alternate within a stage");
  half8 af[2][T::MB], bf[2][T::NB];
  bool ok = true;
  if (S > 0) {
    ok = wait_geq(full, 1u, limit);
    if (trace && wave == 0 && lane == 0) trace[2] = wall_clock64();
    read_step(ring, 0, af[0], bf[0]);
  }
  for (int i = 0; i < S; ++i) {
    const lds_char* const slot = ring + (i % RING) * T::SLOT_BYTES;
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s) {
      const int cur = s & 1;
      if (s + 1 < T::KSTEPS) {
        read_step(slot, s + 1, af[cur ^ 1], bf[cur ^ 1]);
      } else {
        // every operand of stage i is in registers: release its slot first
        // (with one slot, stage i+1 can only land after that)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) store_counter(released + 4 * wave, (uint32_t)(i + 1));
        if (trace && wave == 0 && lane == 0) trace[i * TRACE_FIELDS + 3] = wall_clock64();
        if (i + 1 < S) {
          ok = ok && wait_geq(full, (uint32_t)(i + 2), limit);
          if (trace && wave == 0 && lane == 0) trace[(i + 1) * TRACE_FIELDS + 2] = wall_clock64();
          read_step(ring + ((i + 1) % RING) * T::SLOT_BYTES, 0, af[0], bf[0]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
          acc[mb][nb] = mfma16(bf[cur][nb], af[cur][mb], acc[mb][nb]);
    }
    if (trace && wave == 0) {
      // MFMAs retire in order: reading the last one's result waits for all
      float last;
      asm volatile("v_mov_b32 %0, %1" : "=v"(last) : "v"(acc[T::MB - 1][T::NB - 1][15]));
      asm volatile("" ::"v"(last));
      if (lane == 0) trace[i * TRACE_FIELDS + 4] = wall_clock64();
    }
  }

  // Epilogue: lane (l32, hh) of block (mb, nb) holds row m = l32 and
  // columns 8*g + 4*hh .. +3 in registers 4g .. 4g+3.
#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb) {
    const int m = m0 + wm * (TM / 2) + 32 * mb + l32;
    if (m < p.M) {
      _Float16* crow = p.c + (size_t)m * p.N;
#pragma unroll
      for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * (TN / 2) + 32 * nb + 8 * g + 4 * hh;
          if (n < p.N) {
            half4 w = {(_Float16)acc[mb][nb][4 * g + 0], (_Float16)acc[mb][nb][4 * g + 1],
                       (_Float16)acc[mb][nb][4 * g + 2], (_Float16)acc[mb][nb][4 * g + 3]};
            *reinterpret_cast<half4*>(crow + n) = w;
          }
        }
    }
  }
  if (trace && wave == 0 && lane == 0) {
    trace[S * TRACE_FIELDS + 1] = wall_clock64();
    trace[S * TRACE_FIELDS + 2] = (unsigned long long)t;
    trace[S * TRACE_FIELDS + 3] = 0;
    trace[S * TRACE_FIELDS + 4] = 0;
  }
  if (!ok && p.status && lane == 0) *p.status = 1;
}

}  // namespace wsgemm
