// gfx950 matrix-core helpers: bf16 32x32x16 MFMA fragments and LDS swizzles.
//
// v_mfma_f32_32x32x16_bf16, D[i][j] += sum_k A[i][k] B[k][j] over a 64-lane wave
// (l32 = lane % 32, hi = lane / 32):
//   A operand: lane holds A[l32][8*hi + 0..7]      (8 bf16)
//   B operand: lane holds B[8*hi + 0..7][l32]      (8 bf16)
//   D (16 fp32 per lane): lane holds D[row_of(r, hi)][l32], r = 0..15,
//   row_of(r, hi) = 8*(r/4) + 4*hi + r%4.
// Any permutation of the 16 k slots works as long as A and B agree; the
// kernels use that to feed an accumulator straight back in as a B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int row_of(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ __forceinline__ __bf16 to_bf(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float from_bf(__bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ __bf16 bits_to_bf(uint16_t u) { return __builtin_bit_cast(__bf16, u); }
__device__ __forceinline__ uint16_t bf_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

__device__ __forceinline__ bf16x8_t pack8(const float (&f)[8]) {
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = to_bf(f[j]);
  return r;
}

__device__ __forceinline__ bf16x8_t cat44(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// XOR swizzle of 8-element (16-byte) granules inside a row of a bf16 LDS matrix
// with NCOL columns: element (row, col) lives at row*NCOL + swz(row, col).  A
// run of up to 8 elements starting at a multiple of 4 stays inside one granule.
// gfx950's LDS has 64 four-byte banks (16 groups of 16 bytes), serves a
// ds_read_b128 16 lanes a cycle and a ds_read_b64_tr_b16 32 lanes a cycle.
// With 16 or more granules per row (rows a multiple of 256 bytes) the key of
// row r is 4 (r % 4) + (r / 4) % 4: sixteen consecutive rows take all sixteen
// keys, so one granule read in 16 rows hits 16 bank groups, and the four
// adjacent granules of four consecutive rows that a transpose read's 32 lanes
// name land in 16 bank groups too.  The key depends on r % 16 only.  With 8
// granules per row the key is 2 (r % 4) + (r / 4) % 2 (r % 8 only).
__device__ __forceinline__ int swz_key8(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int swz_key16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
template <int NCOL>
__device__ __forceinline__ int swz_key(int row) {
  constexpr int ngran = NCOL / 8;
  return ngran >= 16 ? swz_key16(row) : ngran >= 8 ? swz_key8(row) : (row & (ngran - 1));
}
template <int NCOL>
__device__ __forceinline__ int swz(int row, int col) {
  return row * NCOL + (((col >> 3) ^ swz_key<NCOL>(row)) << 3) + (col & 7);
}

// LDS (address space 3) views: 32-bit addresses, so a ds_read / ds_write can
// carry a constant offset of up to 64 KiB next to a per-lane base register.
template <typename T>
using lds_t = __attribute__((address_space(3))) T;

// A pointer into a __shared__ array as an LDS pointer whose value is hidden from
// the optimiser.  Constant offsets added to it stay in the instruction's offset
// field; otherwise the compiler folds the array's own position into them (past
// 64 KiB it no longer fits) and spends an add per access.
template <typename T>
__device__ __forceinline__ lds_t<T>* lds_base(T* p) {
  lds_t<T>* q = (lds_t<T>*)p;
  asm volatile("" : "+v"(q));
  return q;
}

// The value of x, hidden from the optimiser.  Lane indices re-derived through it
// at the top of a loop body make the LDS addresses built from them loop-variant,
// so they are formed where they are used instead of being hoisted out of the
// loop and parked in (accumulation) registers or scratch for the whole loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

}  // namespace ttt
