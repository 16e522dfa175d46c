// Device-side helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace ba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ u16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u16(u >> 16);
}

// two floats -> packed bf16x2 (lo = a, hi = b), round to nearest even
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 32x32x16 bf16 matrix-core product, fp32 accumulate.
// Operand lane layout (wave64, lane l, i = l % 32, h = l / 32):
//   A (32 x 16): lane holds A[i][8h .. 8h+7]
//   B (16 x 32): lane holds B[8h .. 8h+7][i]
//   C (32 x 32): lane holds C[8(v/4) + 4h + v%4][i] in element v = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Key permutation inside a group of 16 keys used by every operand that is
// contracted over keys (or queries) after coming out of an MFMA C register:
// slot s of the group holds key kslot16(s), so that lane half h feeds slots
// 8h..8h+7 straight from its C registers v = 0..7 (keys 4h+0..3, 8+4h+0..3).
__device__ __forceinline__ int kslot16(int s) {
  return (s & 3) + ((s >> 3) << 2) + (((s >> 2) & 1) << 3);
}

__device__ __forceinline__ float wave_shfl_xor32(float x) { return __shfl_xor(x, 32, 64); }

}  // namespace ba

namespace ba {

// LDS row strides (bf16 elements), padded against bank conflicts.
constexpr int kNatStride = 136;  // [row][d] tiles: 128 + 8
constexpr int kTrStride = 72;    // [d][slot] tiles of 64 slots: 64 + 8

// Transpose an 8 (rows, in kslot16 order) x 4 (d) block of bf16 values held
// as eight u32x2 (one row each) and store it as 4 LDS rows of 8 slots.
__device__ __forceinline__ void store_t8x4(const u32x2 (&v)[8], u16 *dst_row0, int stride) {
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    u32x4 w;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = (dd < 2) ? v[2 * p].x : v[2 * p].y;
      const uint32_t b = (dd < 2) ? v[2 * p + 1].x : v[2 * p + 1].y;
      w[p] = (dd & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<u32x4 *>(dst_row0 + dd * stride) = w;
  }
}

}  // namespace ba
