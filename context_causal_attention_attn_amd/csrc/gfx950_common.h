// Vector types, LDS tile addressing and wavefront helpers shared by the
// gfx950 share kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

// Row-major LDS tile of bf16 rows of W elements whose 16-byte chunks are
// XOR-swizzled by row: 16 consecutive rows reading the same chunk (MFMA
// A/B operand reads) and 4 rows x 64 contiguous bytes (transpose reads) both
// spread over the banks.
template <int W>
struct Tile {
  static constexpr int NC = W / 8;
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (NC >= 16) {
      return ((row & 3) * (NC / 4) + ((row >> 2) & (NC / 4 - 1))) & (NC - 1);
    } else if constexpr (NC == 8) {
      return ((row & 3) * 2 + ((row >> 2) & 1)) & 7;
    } else {
      return (row >> 1) & (NC - 1);
    }
  }
  __device__ static __forceinline__ int chunk_off(int row, int c) {
    return row * W + ((c ^ swz(row)) << 3);
  }
  __device__ static __forceinline__ int elem_off(int row, int col) {
    return chunk_off(row, col >> 3) + (col & 7);
  }
};

// Row-major LDS tile for the 16x16x32 kernels, read both ways: as rows (16
// consecutive rows, one 16-byte chunk each: an A/B operand) and by
// transposes (8 consecutive rows x 16 columns: a contraction down the rows).
// The chunk swizzle 2*(row mod 8) + (row/8 mod 2) -- 2*((row/2) mod 4) +
// (row/8 mod 2) for 64-element rows, two per bank line -- is a permutation
// over any 16 aligned rows and gives the 8 rows' 2 chunks of any 16-column
// block 16 distinct bank groups, so neither read has bank conflicts. It
// repeats every 16 rows.
template <int W>
struct Tile16 {
  static constexpr int NC = W / 8;
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (NC >= 16) {
      return (2 * (row & 7) + ((row >> 3) & 1)) & (NC - 1);
    } else {
      return (2 * ((row >> 1) & 3) + ((row >> 3) & 1)) & (NC - 1);
    }
  }
  __device__ static __forceinline__ int chunk_off(int row, int c) {
    return row * W + ((c ^ swz(row)) << 3);
  }
  __device__ static __forceinline__ int elem_off(int row, int col) {
    return chunk_off(row, col >> 3) + (col & 7);
  }
};

// Two transpose reads (ds_read_b64_tr_b16) forming one 8 x bf16 MFMA operand
// whose contraction index runs down `rows` of a row-major tile: lane l of the
// wavefront gets column (col0 + 16*((l>>4)&1) + (l&15)) at the 8 rows
// {r0 + 4*(l>>5) + e, r0 + 8 + 4*(l>>5) + e : e = 0..3}, matching the
// row order of a 32x32 MFMA accumulator's register blocks.
template <int W>
__device__ __forceinline__ bf16x8 tr_operand(const __bf16 *tile, int r0, int col0, int lane) {
  const int row = r0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + Tile<W>::elem_off(row, col)));
  const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + Tile<W>::elem_off(row + 8, col)));
  const i16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, a);
}

// Per-lane offsets of the two transpose reads of tr_operand for every 32-wide
// column block, computed once. A block of rows starting at a multiple of 16
// only adds a constant (the swizzle depends on the row modulo 16).
template <int W>
struct TrOffsets {
  static constexpr int NB = W / 32;
  int off[2][NB];
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
        off[u][cb] = Tile<W>::elem_off(8 * u + 4 * (lane >> 5) + ((lane & 15) >> 2),
                                        32 * cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  }
  // Operand of rows [r16, r16+16) (r16 a multiple of 16), column block cb.
  __device__ __forceinline__ bf16x8 read(const __bf16 *tile, int r16, int cb) const {
    const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + off[0][cb] + r16 * W));
    const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + off[1][cb] + r16 * W));
    const i16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, a);
  }
};

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until every outstanding vector-memory load of this wavefront has
// returned (s_waitcnt vmcnt(0); expcnt/lgkmcnt left unconstrained). Used once
// after the loads of register-resident operands, so that the compiler's
// wait-count bookkeeping does not carry them into the main loop, where it
// would otherwise wait on the in-flight prefetch of later tiles.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Round 16 floats to bf16 (nearest-even) into two MFMA operands, element i
// going to lane-element i % 8 of operand i / 8; one conversion per pair.
__device__ __forceinline__ void to_bf16_operands(const float (&v)[16], bf16x8 (&o)[2]) {
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const bf16x2 t = __builtin_convertvector((f32x2){v[j], v[j + 1]}, bf16x2);
    o[j >> 3][j & 7] = t[0];
    o[j >> 3][(j & 7) + 1] = t[1];
  }
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D (16x16) += A (16x32) B (32x16). Lane l holds A row l%16 and B column l%16
// at contraction slots 8*(l/16) .. +7, and D column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum and max over the four lanes that hold the same accumulator column
// (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

template <int N>
using IC = std::integral_constant<int, N>;

// Value of lane N of this lane's row of 16 lanes (DPP row_newbcast); used as
// an operand, it folds into the consuming instruction.
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(N >= 0 && N < 16, "lane within a row of 16");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xF, 0xF, false));
}

// Calls f(IC<0>{}), ..., f(IC<N-1>{}) in order (compile-time loop index).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<N, I + 1>(f);
  }
}

}  // namespace cpattn
