// Device-side building blocks shared by the forward and backward kernels (gfx950 only).
//
// MFMA operand/accumulator layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16},
// wave64, lane l, c = l % 32, g = l / 32):
//   A (32 x 16, row m, column k):  lane l holds A[c][g*8 + j] in slot j = 0..7
//   B (16 x 32, row k, column n):  lane l holds B[g*8 + j][c] in slot j = 0..7
//   C (32 x 32 fp32):              lane l holds C[(i/4)*8 + g*4 + i%4][c] in register i = 0..15
// Because an MFMA sums over k, any permutation of k applied to both A and B gives the
// same product; the kernels use that freedom to chain accumulators into operands.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Placed after a lambda's parameter list: the kernels build their loop bodies from lambdas
// that capture register arrays by reference, which only stay in registers when every call
// is inlined.
#define FA_INL __attribute__((always_inline))

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- element types

struct Bf16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two floats -> packed pair, round to nearest even (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  // acc + lo(w) + hi(w) in one instruction (v_dot2c_f32_bf16 against (1, 1)).
  static __device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  // acc + lo(w) + hi(w) in one instruction (v_dot2c_f32_f16 against (1, 1)).
  static __device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
  }
};

// ---------------------------------------------------------------- global memory

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_if(const uint16_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? ld16(p) : z;
}

// ---------------------------------------------------------------- scheduling

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Remap the hardware
// id so that consecutive logical jobs (the tiles of one head, which stream the same
// K/V) run on the same XCD and share its L2.  A bijection for any grid size.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  constexpr int NXCD = 8;
  const int q = nblk / NXCD, r = nblk % NXCD;
  const int xcd = bid % NXCD, slot = bid / NXCD;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Within an XCD the dispatcher also deals workgroups to its four shader engines in turn and
// strictly in order: a workgroup waits for a free CU on its own engine and holds back every
// later one.  Where tiles carry unequal work (causal grids that run in several rounds), the
// four workgroups of consecutive slots should carry about the same work, or the lighter ones'
// CUs idle until the heaviest one's engine frees a CU.  This variant assigns each XCD the same
// jobs as xcd_remap, but when its range holds h > 1 whole heads of `per_head` jobs each, slot s
// takes job s / h of head s % h: the heads advance together, and four consecutive slots span
// at most two neighbouring tiles instead of four.
__host__ __device__ __forceinline__ int xcd_remap_interleaved(int bid, int nblk, int per_head) {
  constexpr int NXCD = 8;
  const int q = nblk / NXCD, r = nblk % NXCD;
  const int xcd = bid % NXCD, slot = bid / NXCD;
  const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  const int len = xcd < r ? q + 1 : q;
  if (base % per_head != 0 || len % per_head != 0) return base + slot;
  const int h = len / per_head;
  return base + (slot % h) * per_head + slot / h;
}

// Order of a head's causal tiles (work grows linearly with the tile index).  idx counts the
// head's jobs in dispatch order.  When the whole grid is resident at once (`snake`),
// consecutive heads alternate heaviest-first and lightest-first, so the two workgroups a CU
// receives from consecutive heads add up to about the same work on every CU.  Otherwise the
// grid runs in several rounds and heaviest-first lets the dispatcher balance as slots free up.
__host__ __device__ __forceinline__ int causal_tile(int idx, int head, int n, int snake) {
  return (snake && (head & 1)) ? idx : n - 1 - idx;
}
// Whole grid resident at once: every workgroup has a slot on some CU from the start.
inline bool grid_fits(long long blocks, int per_cu) { return blocks <= 256LL * per_cu; }

// ---------------------------------------------------------------- LDS tiles
//
// A tile of R rows x W 16-bit columns (W = 64 or 128) is stored as W/32 "slices" of
// R rows x 32 columns; a slice row is 64 bytes (four 16-byte chunks) and four rows share a
// 256-byte bank line.  The chunk index is XORed with bits 2..3 of the row.  This makes both
// access patterns used on tiles free of bank conflicts (64 banks x 4 bytes):
//   * 16-byte reads/writes by 16 lanes on 16 distinct rows (mod 16), same column;
//   * ds_read_b64_tr_b16 by 32 lanes on 4 consecutive rows x 32 consecutive columns;
// and it keeps every compile-time part of an address additive: for rows rb + lr (rb a
// multiple of 16) and columns cb + lc (cb a multiple of 32, lc < 32),
//   sl_off(rb + lr, cb + lc) = sl_off(rb, cb) + sl_off(lr, lc),
// so a lane computes its offsets once and every read uses an immediate offset.
template <int R>
__device__ __forceinline__ uint32_t sl_off(uint32_t r, uint32_t col) {
  return (col >> 5) * (uint32_t)(R * 64) + r * 64u + ((((col >> 3) & 3u) ^ ((r >> 2) & 3u)) << 4) +
         (col & 7u) * 2u;
}

// Inverse for 16-byte chunks: (row, column) of the chunk stored at 16-byte position P.  The
// direct global->LDS loads write lane l's 16 bytes at base + 16*l, so lane l of the load that
// fills positions [64*i, 64*i + 64) fetches the chunk that belongs at position 64*i + l.
template <int R>
__device__ __forceinline__ void sl_pos_to_rc(uint32_t P, int& row, int& col) {
  const uint32_t slice = P / (uint32_t)(R * 4), q = P % (uint32_t)(R * 4);
  const uint32_t r = q >> 2, pc = q & 3u;
  row = (int)r;
  col = (int)(slice * 32u + ((pc ^ ((r >> 2) & 3u)) << 3));
}

// Direct global -> LDS copies go through a buffer resource (buffer_load_dword{,x4} ... lds):
// every active lane fetches BYTES from base + voff + soff and lane l's data lands at
// lds_base + BYTES * l.  Completion is tracked by vmcnt only.  Bytes at or past
// `bytes` (the resource's extent) read as zero, so ragged tails need no clamping.  (The
// global_load_lds form would do the same copy, but the compiler treats it as a flat access
// that may touch LDS and then makes every later LDS-read wait drain all outstanding LDS
// reads, which defeats operand prefetching while a copy is in flight.)
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes make_bufres(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit data, the gfx9-family default for loads.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(BufRes res, uint32_t voff, uint32_t soff, char* lds_base) {
  static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte direct loads");
  auto* dst = (__attribute__((address_space(3))) void*)lds_base;
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, dst, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, dst, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ u32x4 lds_ld128(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void lds_st128(char* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Row-major output tiles staged through LDS.  In the accumulator layouts a store instruction
// covers 2 to 8 bytes of each of 32 rows per lane; with every CU storing its tile at about the
// same moment such partial-line writes cost several microseconds per workgroup.  A wave
// therefore writes its rows into a private LDS region (rows of RB bytes, their 16-byte chunks
// XOR-swizzled by the row index, so that column-wise writes over consecutive rows and
// row-wise reads spread over the banks) and stores them back as 16 bytes per lane, 1 KB of
// consecutive rows per instruction.
template <int RB>
__device__ __forceinline__ uint32_t stage_off(int r, int ch) {
  constexpr int CH = RB / 16;  // 16-byte chunks per row
  return (uint32_t)(r * RB + ((ch ^ (r & (CH - 1))) << 4));
}
// 16-bit rows of HD columns: lane (c, g) puts row r's columns db*32 + i4*8 + g*4 .. +3
// (two packed pairs, w[db][i4]).
template <int HD>
__device__ __forceinline__ void stage_row(char* region, int r, int g, const u32x2 (&w)[HD / 32][4]) {
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *reinterpret_cast<u32x2*>(region + stage_off<HD * 2>(r, db * 4 + i4) + g * 8) = w[db][i4];
}
// Copies the region's first R rows to dst, whose rows are STRIDE bytes apart (a staged row may
// be part of a destination row); rows >= n_valid are skipped.
template <int RB, int R, int STRIDE = RB>
__device__ __forceinline__ void store_staged(const char* region, void* dst, int n_valid, int lane) {
  constexpr int CH = RB / 16, RPI = 64 / CH;  // chunks per row, rows per instruction
  static_assert(R % RPI == 0, "whole instructions");
#pragma unroll
  for (int k = 0; k < R / RPI; ++k) {
    const int r = k * RPI + lane / CH, ch = lane % CH;
    const u32x4 v = lds_ld128(region + stage_off<RB>(r, ch));
    // (non-temporal: the output is not read again here; 0.3-1.2% faster forward at N >= 4096)
    if (r < n_valid) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<char*>(dst) + (size_t)r * STRIDE + ch * 16));
  }
}

// Lane offsets of the transposed-operand read (see lds_tr8): rows lr and lr + 4, column lc.
struct TrLane {
  uint32_t r0, r4;
};
__device__ __forceinline__ TrLane tr_lane(int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int lr = (grp >> 1) * 8 + (i >> 2);
  const int lc = (grp & 1) * 16 + (i & 3) * 4;
  return TrLane{sl_off<16>(lr, lc), sl_off<16>(lr + 4, lc)};
}

// Transposed operand fragment at tile position p (= tile + sl_off(rowbase, colbase), rowbase
// a multiple of 16, colbase a multiple of 32): slot j of lane l receives
// T[rowbase + g*8 + j][colbase + c] (c = l % 32, g = l / 32), eight elements down a column,
// as an MFMA operand needs when the contraction runs along the tile's rows.  Two
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the 8-byte
// words addressed by lanes 4r + i/4 (r = 0..3), in slot r.
__device__ __forceinline__ u32x4 lds_tr8(const char* p, TrLane t) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + t.r0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + t.r4));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  u32x4 r = {ua[0], ua[1], ub[0], ub[1]};
  return r;
}

// Row permutation applied to the A-operand rows of an S = X Y^T product (swap bits 2
// and 3 of the row index).  With it, accumulator register i of lane (c, g) holds row
// (i/8)*16 + g*8 + i%8, so registers 8t..8t+7 are eight consecutive rows: exactly the
// k-slots of an operand whose contraction runs over those rows.
__device__ __forceinline__ int perm_rows(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// ---------------------------------------------------------------- cross-lane

// Value of lanes l and l ^ 32 combined, via v_permlane32_swap (swaps the upper half of
// the first operand with the lower half of the second).
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- software pipelining

// Runs compute(i, operands_i) for i = 0..NSTEP-1 with the LDS reads of step i + DIST issued
// before step i computes (a register ring of DIST + 1 operand sets).  The fences pin this
// order, so the waits the compiler inserts are partial (LDS reads retire in order) and a
// wave keeps DIST steps of reads in flight behind its MFMAs.
template <int NSTEP, int DIST, typename LoadF, typename ComputeF>
__device__ __forceinline__ void pipelined(LoadF&& load, ComputeF&& compute) {
  using Ops = decltype(load(0));
  Ops ring[DIST + 1];
#pragma unroll
  for (int i = 0; i < DIST && i < NSTEP; ++i) ring[i] = load(i);
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (i + DIST < NSTEP) ring[(i + DIST) % (DIST + 1)] = load(i + DIST);
    __builtin_amdgcn_sched_barrier(0);
    compute(i, ring[i % (DIST + 1)]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- synchronisation

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations, which include
// its direct global->LDS loads (the LDS-scoped release fence waits for those too, vmcnt(0)),
// but not for its global stores or ordinary loads.  (HIP's __syncthreads also drains every
// outstanding global load, store and atomic.)  Where later tiles' direct loads should stay
// in flight across the barrier, dma_barrier below is the one to use.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Written-out MFMAs (v_mfma_f32_32x32x16 bf16/fp16), for kernels that keep accumulators or
// stationary operands in AGPRs while other MFMA results land in VGPRs for the VALU: the
// compiler picks one register form for all MFMAs of a kernel, so such a mix is inline
// assembly.  The compiler does not see these as MFMAs and inserts no wait states for them, so
// a sequence of them carries its own where needed (CDNA3/CDNA4 dependency rules): kNopBefore
// waits 2 for VALU writes of its operands (s_nop 1), kNopAfter waits 24 (three s_nop 7) before
// anything else may touch a result, kNopBoth does both (an 8-pass XDL result needs at most 19 before a VALU,
// v_accvgpr or memory access).  The waits are in the same statement as the MFMA, so no
// instruction the compiler places around it can fall inside the window.  A and B are read when
// an MFMA issues, and an exactly overlapping accumulator chains without wait states.  The
// library's tests check the windows on the compiled code.
enum { kNopNone, kNopBefore, kNopAfter, kNopBoth };
#define FA_MFMA_ASM(NOP, TEXT, OUT, ...)                                                      \
  do {                                                                                        \
    if constexpr (NOP == kNopBefore)                                                          \
      asm volatile("s_nop 1\n\t" TEXT : OUT : __VA_ARGS__);                                   \
    else if constexpr (NOP == kNopAfter)                                                      \
      asm volatile(TEXT "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : OUT : __VA_ARGS__);             \
    else if constexpr (NOP == kNopBoth)                                                       \
      asm volatile("s_nop 1\n\t" TEXT "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : OUT : __VA_ARGS__); \
    else                                                                                      \
      asm volatile(TEXT : OUT : __VA_ARGS__);                                                 \
  } while (0)
template <typename TR, int NOP>  // acc (AGPR) += a b
__device__ __forceinline__ void mfma_av(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (std::is_same<TR, F16>::value)
    FA_MFMA_ASM(NOP, "v_mfma_f32_32x32x16_f16 %0, %1, %2, %0", "+a"(acc), "v"(a), "v"(b));
  else
    FA_MFMA_ASM(NOP, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0", "+a"(acc), "v"(a), "v"(b));
}
template <typename TR, int NOP>  // acc (VGPR) += a b (b in AGPRs)
__device__ __forceinline__ void mfma_va(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (std::is_same<TR, F16>::value)
    FA_MFMA_ASM(NOP, "v_mfma_f32_32x32x16_f16 %0, %1, %2, %0", "+v"(acc), "v"(a), "a"(b));
  else
    FA_MFMA_ASM(NOP, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0", "+v"(acc), "v"(a), "a"(b));
}
template <typename TR, int NOP>  // acc (VGPR) = a b (b in AGPRs)
__device__ __forceinline__ void mfma_va0(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (std::is_same<TR, F16>::value)
    FA_MFMA_ASM(NOP, "v_mfma_f32_32x32x16_f16 %0, %1, %2, 0", "=&v"(acc), "v"(a), "a"(b));
  else
    FA_MFMA_ASM(NOP, "v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0", "=&v"(acc), "v"(a), "a"(b));
}
#undef FA_MFMA_ASM
// Ordering point for the registers of `r`: each is an operand here, so no access to them
// moves across it.  With `nop`, two wait states follow (after VALU or v_accvgpr writes of `r`,
// before MFMAs read it).  The scheduler also keeps live ranges short around these points.
template <typename T, int A, int B>
__device__ __forceinline__ void reg_fence(T (&r)[A][B], bool agpr, bool nop) {
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (agpr)
        asm volatile("" : "+a"(r[i][j]));
      else
        asm volatile("" : "+v"(r[i][j]));
    }
  if (nop) asm volatile("s_nop 1" ::: "memory");
}

// Workgroup barrier that drains only this wave's LDS operations, even while direct
// global->LDS loads are still in flight (lds_barrier's fence would also wait for those,
// since they write LDS).  For hand-offs of LDS data written with ordinary LDS stores; the
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_store_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier for tiles filled by direct loads.  The caller has already waited (vmcnt)
// for its own share of the tile it needs next; this drains the wave's LDS reads (so that a
// buffer may be refilled after the barrier) and synchronises, without also waiting for direct
// loads still in flight for later tiles, which an LDS-scoped fence would do.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N): wait until at most N of this wave's vector-memory operations are
// outstanding.  On gfx9-family targets loads, stores, atomics and direct-to-LDS loads share
// this counter and retire in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace fa
