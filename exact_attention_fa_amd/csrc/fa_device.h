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

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

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
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  constexpr int NXCD = 8;
  const int q = nblk / NXCD, r = nblk % NXCD;
  const int xcd = bid % NXCD, slot = bid / NXCD;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// ---------------------------------------------------------------- LDS tiles
//
// A tile is a row-major array of 16-bit elements with ROW (64 or 128) elements per row,
// packed into 256-byte bank lines (one row of 128, or two rows of 64).  The 16-byte
// chunk index inside a bank line is XOR-swizzled with a function of the line index so
// that both access patterns used on tiles are free of bank conflicts:
//   * ds_read_b128 / ds_write_b128 by 16 lanes on 16 distinct rows (mod 16), same chunk;
//   * ds_read_b64_tr_b16 by 32 lanes on 4 consecutive rows and 4 consecutive chunks.
template <int ROW>
__device__ __forceinline__ uint32_t lds_off(uint32_t r, uint32_t c) {
  static_assert(ROW == 64 || ROW == 128, "tile rows hold 64 or 128 elements");
  if constexpr (ROW == 128) {
    const uint32_t f = ((r & 3u) << 2) | ((r >> 2) & 3u);
    return r * 256u + ((c ^ f) << 4);
  } else {
    const uint32_t line = r >> 1;
    const uint32_t slot = ((r & 1u) << 3) | c;
    const uint32_t f = ((line & 1u) << 2) | ((line >> 1) & 3u);
    return line * 256u + ((slot ^ f) << 4);
  }
}

template <int ROW>
__device__ __forceinline__ void lds_write8(char* tile, int row, int col, u32x4 v) {
  *reinterpret_cast<u32x4*>(tile + lds_off<ROW>(row, col >> 3)) = v;
}

// Eight consecutive elements T[row][col .. col+7] (col a multiple of 8).
template <int ROW>
__device__ __forceinline__ u32x4 lds_read8(const char* tile, int row, int col) {
  return *reinterpret_cast<const u32x4*>(tile + lds_off<ROW>(row, col >> 3));
}

// Transposed operand fragment: slot j of lane l receives T[rowbase + g*8 + j][colbase + c]
// (c = l % 32, g = l / 32), i.e. eight elements down a column, as the MFMA A or B operand
// wants when the contraction index runs along the tile's rows.  Uses two
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the
// 8-byte words addressed by lanes 4r + i/4 (r = 0..3), in slot r.
template <int ROW>
__device__ __forceinline__ u32x4 lds_read_tr8(const char* tile, int rowbase, int colbase, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int row = rowbase + (grp >> 1) * 8 + (i >> 2);
  const int col = colbase + (grp & 1) * 16 + (i & 3) * 4;
  const uint32_t sub = (uint32_t)(col & 4) << 1;  // byte offset of the word inside its chunk
  const lds_s16x4* p0 = (const lds_s16x4*)(tile + lds_off<ROW>(row, col >> 3) + sub);
  const lds_s16x4* p1 = (const lds_s16x4*)(tile + lds_off<ROW>(row + 4, col >> 3) + sub);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
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

}  // namespace fa
