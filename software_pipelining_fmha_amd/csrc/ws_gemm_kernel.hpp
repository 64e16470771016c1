// Warp-specialised fp16 GEMM for gfx950 (MI355X, CDNA4): C = A B with A
// [M][K], B [K][N] and C [M][N] row-major binary16, fp32 accumulation.
//
// Structure (performance-model page for warp-specialised kernels, sections
// "Warp specialization kernel structure" and "Algorithm 1"): each workgroup
// computes one T_M x T_N output tile in S = ceil(K / T_K) stages, with two
// kinds of wave.
// - DMA waves (DMA_WAVES of them, each an equal share of every stage) move
//   each stage's A tile (T_M x T_K) and B tile (T_K x T_N) from HBM into a
//   ring of RING slots in LDS by LDS-DMA (buffer_load ... lds). They wait
//   while the ring is full.
// - Four MATH waves (each a quarter of the tile) read the stage's operands
//   from LDS into registers, run the fp16 MFMAs, release the slot, and
//   finally store their part of C.
// The page's wait()/signal() semaphores are counters in LDS: one `full`
// counter per DMA wave (stages whose share has landed) and one `released`
// counter per MATH wave (stages that wave has finished reading). A stage is
// in once every DMA wave's count covers it; a DMA wave reuses a slot once
// the slowest MATH wave has released it. Waves run independently, so a
// single summed count could be reached while one wave still reads the slot.
// Waiting is polling with s_sleep. Every poll loop is bounded, and a wave
// that gives up reports it through the status word, so no wave can wait
// forever.
//
// Each DMA wave keeps up to two stages of its share in flight. Its share
// has landed once the wave's vmcnt shows its loads done (loads complete in
// issue order). Before it blocks on a full ring it signals everything it
// has issued, so the MATH waves can always drain the ring. One wave can
// keep only 63 loads (63 KB) in flight, and at L2 latency that caps how
// fast it fills the ring: four DMA waves are what let the 256 x 128 tile
// run at the matrix cores' pace.
//
// gfx950 mapping. The product is formed transposed, C^T = B^T A^T, with
// v_mfma_f32_32x32x16_f16: the B^T operand (rows n, 8 consecutive k per
// lane) comes from the row-major B tile through ds_read_b64_tr_b16, and the
// A^T operand (8 consecutive k of one row m per lane) is one 16-byte read
// of the row-major A tile. Each accumulator lane then holds one row m and 4
// consecutive columns n per register group, stored as 8-byte writes.
// Both LDS tiles are swizzled in 16-byte chunks so that these reads hit
// distinct banks; the DMA waves write that layout directly by choosing each
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
// [0] DMA wave 0 starts issuing stage i, [1] DMA wave 0 sees its share of
// stage i landed and signals it, [2] MATH wave 0 starts stage i, [3] MATH wave 0 releases
// stage i's slot, [4] MATH wave 0's MFMAs of stage i have finished. Row S:
// [0] workgroup start, [1] MATH wave 0 done with its stores, [2] the tile
// id, [3] and [4] 0. Only a traced launch waits for [4] (a register read of
// the stage's last accumulator), so only it is slowed by it.
constexpr int TRACE_FIELDS = 5;
// DMA waves, each moving an equal share of every stage, and four MATH waves.
constexpr int DMA_WAVES = 4;
constexpr int GEMM_THREADS = (4 + DMA_WAVES) * 64;

template <int TM, int TN, int TK, int RING>
struct GemmTile {
  static constexpr int MATH_WAVES = 4;
  static constexpr int THREADS = GEMM_THREADS;
  static constexpr int MB = TM / 64;       // 32-row blocks per MATH wave (a wave has TM/2 rows)
  static constexpr int NB = TN / 64;       // 32-column blocks per MATH wave
  static constexpr int KSTEPS = TK / 16;   // MFMA k-steps per stage
  static constexpr int CA = TK / 8;        // 16-byte chunks per A tile row
  static constexpr int CB = TN / 8;        // 16-byte chunks per B tile row
  // A tile: chunk c of row r sits at chunk c ^ a_swz(r). ds_read_b128 serves
  // 16 lanes (16 consecutive rows, one chunk) per pass, and the LDS banks
  // span 256 bytes: with 128-byte rows, rows r and r + 8 share banks unless
  // the swizzle differs across them, so it follows r / 2 there.
  static constexpr __device__ __host__ int a_swz(int r) { return CA == 8 ? (r >> 1) & 7 : r & 15; }
  static constexpr int A_BYTES = TM * TK * 2;
  static constexpr int B_BYTES = TK * TN * 2;
  static constexpr int SLOT_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024;  // 1 KB per wave-wide LDS-DMA
  static constexpr int B_LOADS = B_BYTES / 1024;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int A_SHARE = A_LOADS / DMA_WAVES, B_SHARE = B_LOADS / DMA_WAVES;
  static constexpr int SHARE = A_SHARE + B_SHARE;  // loads per DMA wave and stage
  static constexpr int RING_BYTES = RING * SLOT_BYTES;
  // At least 82 KB, so one workgroup occupies a CU (the model's unit).
  static constexpr int LDS_BYTES = (RING_BYTES + 64 > 82 * 1024) ? RING_BYTES + 64 : 82 * 1024;
  static_assert(TM == 64 || TM == 128 || TM == 256, "T_M");
  static_assert(TN == 64 || TN == 128, "T_N");
  static_assert(TK == 64 || TK == 128, "T_K");
  static_assert(RING >= 1 && RING <= 4, "ring depth");
  static_assert(A_LOADS % DMA_WAVES == 0 && B_LOADS % DMA_WAVES == 0, "equal shares");
  static_assert(SHARE <= 63, "vmcnt holds 63");
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

// The DMA waves' `full` counters, read together by one LDS read.
static_assert(DMA_WAVES == 2 || DMA_WAVES == 4, "one 8- or 16-byte read of the counters");
typedef uint32_t FullCounts __attribute__((ext_vector_type(DMA_WAVES)));
// Issue the read; the caller waits for it (lgkmcnt) before using the value.
__device__ __forceinline__ FullCounts read_full(uint32_t addr) {
  FullCounts v;
  if constexpr (DMA_WAVES == 2)
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr));
  else
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ uint32_t min_count(FullCounts v) {
  uint32_t m = v[0];
#pragma unroll
  for (int w = 1; w < DMA_WAVES; ++w) m = min(m, v[w]);
  return m;
}

// Poll the DMA waves' `full` counters until their minimum reaches `target`.
// Inline asm keeps the compiler from waiting on this wave's LDS-DMA before
// the read. Returns false if it gave up after `limit` polls.
__device__ __forceinline__ bool wait_full_geq(const lds_char* cnt, uint32_t target, int limit) {
  for (int n = 0; n < limit; ++n) {
    FullCounts v = read_full(lds_addr(cnt));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v)::"memory");
    if (__builtin_amdgcn_readfirstlane(min_count(v)) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

__device__ __forceinline__ void store_counter(lds_char* cnt, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(cnt)), "v"(v) : "memory");
}

// Read schedule of a MATH wave's k-step (MB x NB MFMA blocks). Read units
// in order: A block 0, B blocks 0 .. NB-1 (two reads each), A blocks
// 1 .. MB-1. MFMA j = (j / NB, j % NB) needs A block j / NB and B block
// j % NB. The next k-step's units go out after the MFMAs, ceil(UNITS / NM)
// per MFMA from the first on.
template <int MB, int NB>
struct GemmUnits {
  static constexpr int NM = MB * NB, UNITS = MB + NB, READS = MB + 2 * NB;
  static constexpr int PER = (UNITS + NM - 1) / NM;
  // reads in units 0 .. u-1
  static constexpr int reads_before_unit(int u) {
    return u <= 0 ? 0 : u <= NB + 1 ? 1 + 2 * (u - 1) : 1 + 2 * NB + (u - NB - 1);
  }
  // reads MFMA j waits for, counted from the k-step's first read
  static constexpr int needed(int j) {
    const int mb = j / NB, nb = j % NB;
    const int ua = mb == 0 ? 0 : NB + mb, ub = 1 + nb;
    const int ea = reads_before_unit(ua + 1), eb = reads_before_unit(ub + 1);
    return ea > eb ? ea : eb;
  }
  // units of the next k-step issued after MFMA j - 1 (before MFMA j)
  static constexpr int first_unit(int j) { return j * PER < UNITS ? j * PER : UNITS; }
  // the same over the last `slots` MFMAs of a stage's last k-step
  static constexpr int first_unit_tail(int j, int slots) {
    return j * ((UNITS + slots - 1) / slots) < UNITS ? j * ((UNITS + slots - 1) / slots) : UNITS;
  }
  static constexpr int issued_before(int j) { return reads_before_unit(first_unit(j)); }
  // LDS operations outstanding after MFMA j's operands when `extra` more
  // were issued after this k-step's reads
  static constexpr int after(int j, int extra) { return READS - needed(j) + extra; }
  // every MFMA needs at least A block 0 and B block 0 (three reads), so a
  // wait never exceeds 2 READS - 3 outstanding operations
  static_assert(2 * READS - 3 <= 15, "waits fit lgkmcnt");
};

template <int TM, int TN, int TK, int RING>
__global__ __launch_bounds__(GEMM_THREADS) void ws_gemm_kernel(GemmParams p) {
  using T = GemmTile<TM, TN, TK, RING>;
  __shared__ __attribute__((aligned(16))) char smem_raw[T::LDS_BYTES];
  lds_char* const ring = (lds_char*)smem_raw;
  lds_char* const full = ring + T::RING_BYTES;   // per DMA wave: stages landed (its share)
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

  static_assert(DMA_WAVES <= 4, "four `full` counters");
  if (tid < 8) {
    store_counter(full + 4 * tid, 0u);  // full[0..3], released[0..3]
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  __syncthreads();

  if (wave >= T::MATH_WAVES) {
    // ---------------- DMA waves ----------------
    // DMA wave dw moves loads dw, dw + DMA_WAVES, ... of each stage's A
    // loads and of its B loads, and counts its own share in full[dw].
    const int dw = wave - T::MATH_WAVES;
    lds_char* const my_full = full + 4 * dw;
    const bool stamp = trace && dw == 0 && lane == 0;
    if (stamp) trace[S * TRACE_FIELDS + 0] = wall_clock64();
    const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(p.a, (uint32_t)p.M * p.K * 2u);
    const __amdgpu_buffer_rsrc_t rb = gemm_rsrc(p.b, (uint32_t)p.K * p.N * 2u);
    // Per load instruction: the global element this lane fetches at k0 = 0,
    // and its column (k for A, n for B) for the bounds test.
    int a_off[T::A_SHARE], a_col[T::A_SHARE];
#pragma unroll
    for (int q = 0; q < T::A_SHARE; ++q) {
      const int j = dw + DMA_WAVES * q;
      const int xx = 64 * j + lane, r = xx / T::CA, pos = xx % T::CA;
      const int c = pos ^ T::a_swz(r);
      a_col[q] = 8 * c;
      a_off[q] = (m0 + r) * p.K + 8 * c;
    }
    int b_off[T::B_SHARE], b_col[T::B_SHARE];
#pragma unroll
    for (int q = 0; q < T::B_SHARE; ++q) {
      const int j = dw + DMA_WAVES * q;
      const int xx = 64 * j + lane, kr = xx / T::CB, pos = xx % T::CB;
      const int c = pos ^ ((T::CB == 16 ? 4 : 2) * (kr & 3));
      b_col[q] = n0 + 8 * c;
      b_off[q] = kr * p.N + n0 + 8 * c;
    }
    bool ok = true, pending = false;
    for (int i = 0; i < S; ++i) {
      if (i >= RING) {
        const uint32_t need = (uint32_t)(i - RING + 1);  // stage i - RING released by all
        if (pending && !wait_min4_geq(released, need, 1)) {
          // The ring is full: signal what is in flight before blocking, so
          // that the MATH waves can drain it.
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (stamp) trace[(i - 1) * TRACE_FIELDS + 1] = wall_clock64();
          if (lane == 0) store_counter(my_full, (uint32_t)i);
          pending = false;
        }
        ok = ok && wait_min4_geq(released, need, limit);
      }
      if (stamp) trace[i * TRACE_FIELDS + 0] = wall_clock64();
      lds_char* const slot = ring + (i % RING) * T::SLOT_BYTES + 1024 * dw;
      const int k0 = i * TK;
#pragma unroll
      for (int q = 0; q < T::A_SHARE; ++q) {
        const int off = (k0 + a_col[q] < p.K) ? 2 * (a_off[q] + k0) : OOB;
        dma16(ra, off, slot + 1024 * DMA_WAVES * q);
      }
#pragma unroll
      for (int q = 0; q < T::B_SHARE; ++q) {
        const int off = (b_col[q] < p.N) ? 2 * (b_off[q] + k0 * p.N) : OOB;
        dma16(rb, off, slot + T::A_BYTES + 1024 * DMA_WAVES * q);
      }
      if (pending) {  // all but stage i's loads have landed: stage i-1 is in
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::SHARE) : "memory");
        if (stamp) trace[(i - 1) * TRACE_FIELDS + 1] = wall_clock64();
        if (lane == 0) store_counter(my_full, (uint32_t)i);
      }
      pending = true;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (S > 0) {
      if (stamp) trace[(S - 1) * TRACE_FIELDS + 1] = wall_clock64();
      if (lane == 0) store_counter(my_full, (uint32_t)S);
    }
    if (!ok && p.status && lane == 0) *p.status = 1;
    return;
  }

  // ---------------- MATH waves ----------------
  constexpr int MB = T::MB, NB = T::NB, KS = T::KSTEPS, NM = MB * NB;
  static_assert(KS % 2 == 0, "k-step buffers alternate; a stage ends on buffer 1");
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  // A^T operand: row m = wm*TM/2 + 32*mb + l32 of the A tile, chunk 2*s + hh
  // of k-step s, stored at chunk ^ a_swz(row). Offsets are slot-relative.
  uint32_t a_off[KS][MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * (TM / 2) + 32 * mb + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) a_off[s][mb] = r * TK * 2 + 16 * ((2 * s + hh) ^ T::a_swz(r));
  }
  // B^T operand by ds_read_b64_tr_b16: in 16-lane group g, lane i reads 4
  // columns (col .. col+3) of k-row 8*(g/2) + i/4 (+ 16 s + 4 q), and
  // receives column 16*(g%2) + i of 4 consecutive k-rows.
  uint32_t b_off[NB];
  {
    const int g = lane >> 4, i = lane & 15;
    const int kr = 8 * (g >> 1) + (i >> 2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * (TN / 2) + 32 * nb + 16 * (g & 1) + 4 * (i & 3);
      const int c = (col >> 3) ^ ((T::CB == 16 ? 4 : 2) * (kr & 3));
      b_off[nb] = T::A_BYTES + kr * TN * 2 + 16 * c + 2 * (col & 7);
    }
  }
  const uint32_t ring_lds = lds_addr(ring);
  const uint32_t full_lds = lds_addr(full);
  const uint32_t released_lds = lds_addr(released + 4 * wave);

  floatx16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // Operands of a k-step, in two buffers (k-steps alternate). Each is read
  // during the previous k-step's MFMAs, unit by unit in the order the MFMAs
  // first need them (A block 0, the B blocks, then A blocks 1 ..); a B unit
  // is two transposing reads. Reads are inline asm with explicit waits: the
  // compiler would otherwise place each read right before its use.
  half8 af[2][MB], bf[2][NB];
  using U = GemmUnits<MB, NB>;
  auto read_unit = [&](int buf, uint32_t slot_lds, int s, int u) __attribute__((always_inline)) {
    if (u == 0 || u > NB) {
      const int mb = u == 0 ? 0 : u - NB;
      asm volatile("ds_read_b128 %0, %1" : "=v"(af[buf][mb]) : "v"(slot_lds + a_off[s][mb]));
    } else {
      const int nb = u - 1;
      shortx4 lo, hi;
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(lo) : "v"(slot_lds + b_off[nb]), "i"(16 * s * TN * 2));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                   : "=v"(hi) : "v"(slot_lds + b_off[nb]), "i"(16 * s * TN * 2 + 4 * TN * 2));
      bf[buf][nb] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // MFMA j of a k-step is block (j / NB, j % NB). `after` = LDS operations
  // issued after the last read it needs.
  auto mfma_waited = [&](int buf, int j, int after) __attribute__((always_inline)) {
    const int mb = j / NB, nb = j % NB;
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(af[buf][mb]), "+v"(bf[buf][nb]) : "n"(after));
    acc[mb][nb] = mfma16(bf[buf][nb], af[buf][mb], acc[mb][nb]);
  };
  auto mfma_ready = [&](int buf, int j) __attribute__((always_inline)) {
    const int mb = j / NB, nb = j % NB;
    acc[mb][nb] = mfma16(bf[buf][nb], af[buf][mb], acc[mb][nb]);
  };

  bool ok = true;
  if (S > 0) {
    ok = wait_full_geq(full, 1u, limit);
    if (trace && wave == 0 && lane == 0) trace[2] = wall_clock64();
#pragma unroll
    for (int u = 0; u < U::UNITS; ++u) read_unit(0, ring_lds, 0, u);
  }
  for (int i = 0; i < S; ++i) {
    const uint32_t slot_lds = ring_lds + (uint32_t)(i % RING) * T::SLOT_BYTES;
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) {
      // k-step s; the reads of k-step s + 1 go between its MFMAs
      const int cur = s & 1;
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_waited(cur, j, U::after(j, U::issued_before(j)));
#pragma unroll
        for (int u = U::first_unit(j); u < U::first_unit(j + 1); ++u) read_unit(cur ^ 1, slot_lds, s + 1, u);
      }
    }
    // Last k-step. A poll of `full` goes out first; once the first half of
    // the MFMAs is issued, every read of this slot has completed: release
    // the slot, check that stage i + 1 has landed (else keep polling), and
    // read its first operands between the remaining MFMAs.
    constexpr int LAST = (KS - 1) & 1, HALF = NM / 2;
    __builtin_amdgcn_sched_barrier(0);
    FullCounts fv = read_full(full_lds);
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_waited(LAST, j, U::after(j, 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fv) ::"memory");
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(af[LAST][mb]));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(bf[LAST][nb]));
    // one lane writes: 64 lanes on one address would serialise on its bank
    if (lane == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(released_lds), "v"((uint32_t)(i + 1)) : "memory");
    if (trace && wave == 0 && lane == 0) trace[i * TRACE_FIELDS + 3] = wall_clock64();
    const bool more = i + 1 < S;
    if (more) {
      if (__builtin_amdgcn_readfirstlane(min_count(fv)) < (uint32_t)(i + 2)) ok = ok && wait_full_geq(full, (uint32_t)(i + 2), limit);
      if (trace && wave == 0 && lane == 0) trace[(i + 1) * TRACE_FIELDS + 2] = wall_clock64();
    }
    const uint32_t next_lds = ring_lds + (uint32_t)((i + 1) % RING) * T::SLOT_BYTES;
#pragma unroll
    for (int j = HALF; j < NM; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_ready(LAST, j);
      if (more) {
#pragma unroll
        for (int u = U::first_unit_tail(j - HALF, NM - HALF); u < U::first_unit_tail(j - HALF + 1, NM - HALF); ++u)
          read_unit(0, next_lds, 0, u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (trace && wave == 0) {
      // MFMAs retire in order: reading the last one's result waits for all
      float last;
      asm volatile("v_mov_b32 %0, %1" : "=v"(last) : "v"(acc[MB - 1][NB - 1][15]));
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
