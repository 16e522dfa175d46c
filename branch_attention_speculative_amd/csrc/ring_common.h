// Pieces shared by the bf16 matrix-core ring kernels: the ring walk over
// (step, chunk) segments and the LDS operand reads.
#pragma once

#include "common.h"

namespace ba {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kRS = 136;  // LDS row stride (bf16) of natural [row][128] tiles

// Two floats -> packed bf16x2 with the hardware round-to-nearest-even convert.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2 r = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight floats -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const float *x) {
  u32x4 w;
#pragma unroll
  for (int p = 0; p < 4; ++p) w[p] = cvt_pk_bf16(x[2 * p], x[2 * p + 1]);
  return as_bf16x8(w);
}

// Natural operand from a row-major LDS tile X[row][col] (row stride kRS):
// lane l takes row row0 + l%32 and the 8 columns col0 + 8*(l/32) .. +7.
// Serves A operands (rows = M, cols = K) and B operands (rows = N, cols = K).
__device__ __forceinline__ bf16x8 lds_nat(const u16 *X, int row0, int col0, int lane) {
  return as_bf16x8(
      *reinterpret_cast<const u32x4 *>(X + (row0 + (lane & 31)) * kRS + col0 + 8 * (lane >> 5)));
}

// Transposed operand from a row-major LDS tile X[k][m] (row stride kRS), for
// a contraction over the tile's rows: the operand element (m, slot s) is
// X[k0 + kslot16(s)][m0 + m]. Two ds_read_b64_tr_b16 per lane: inside each
// 16-lane group, lane j receives element j%4 of the 8-byte chunks addressed
// by lanes 4e + j/4 (e = 0..3), so pointing lane i at row (i/4) and column
// chunk (i%4) hands lane j four consecutive rows of column j.
__device__ __forceinline__ bf16x8 lds_tr(const u16 *X, int k0, int m0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int mb = (g & 1) << 4, h = g >> 1;
  const u16 *p0 = X + (k0 + 4 * h + (i >> 2)) * kRS + m0 + mb + 4 * (i & 3);
  const u16 *p1 = p0 + 8 * kRS;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// ---- ring walk ------------------------------------------------------------

struct Seg {
  int n_hi;      // keys of this chunk visible to the tile's largest bound
  int n_full;    // keys visible to every row of the tile
  int cpos0;     // sequence position of the chunk's first key
  int64_t krow;  // row of the chunk's first key in the [C * N] key array
};

// Segment sg = 2*i + half: ring step i (shard (r - i) mod C), the sequence's
// head (0) or tail (1) chunk inside that shard.
__device__ __forceinline__ Seg seg_info(int sg, const QTile &t, int C, int r, int n_local) {
  const int i = sg >> 1, half = sg & 1;
  int sh = r - i;
  if (sh < 0) sh += C;
  const int chunk = half ? 2 * C - 1 - sh : sh;
  Seg s;
  s.cpos0 = chunk * t.c;
  s.n_hi = min(max(t.p_max - s.cpos0 + 1, 0), t.c);
  s.n_full = min(max(t.p_min - s.cpos0 + 1, 0), t.c);
  s.krow = int64_t(sh) * n_local + t.seq_off + int64_t(half) * t.c;
  return s;
}

template <int BN>
__device__ __forceinline__ void first_block(int &sg, int &j0, Seg &s, const QTile &t, int C, int r,
                                            int n_local) {
  j0 = 0;
  for (sg = 0; sg < 2 * C; ++sg) {
    s = seg_info(sg, t, C, r, n_local);
    if (s.n_hi > 0) return;
  }
}

template <int BN>
__device__ __forceinline__ void next_block(int &sg, int &j0, Seg &s, const QTile &t, int C, int r,
                                           int n_local) {
  j0 += BN;
  if (j0 < s.n_hi) return;
  j0 = 0;
  for (++sg; sg < 2 * C; ++sg) {
    s = seg_info(sg, t, C, r, n_local);
    if (s.n_hi > 0) return;
  }
}

// Load a 64-row x 128-col bf16 block of K or V rows krow + min(j0 + i, n_hi - 1)
// into registers: 256 threads x 4 x 16 bytes.
__device__ __forceinline__ void load_rows64(u32x4 (&R)[4], const u16 *__restrict__ X, const Seg &s,
                                           int j0, int g, int hkv, int tid) {
  const int64_t rs = int64_t(hkv) * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int row = id >> 4, dc = id & 15;
    const int kk = min(j0 + row, s.n_hi - 1);
    R[i] = *reinterpret_cast<const u32x4 *>(X + (s.krow + kk) * rs + g * 128 + dc * 8);
  }
}

__device__ __forceinline__ void store_rows64(const u32x4 (&R)[4], u16 *dst, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int row = id >> 4, dc = id & 15;
    *reinterpret_cast<u32x4 *>(dst + row * kRS + dc * 8) = R[i];
  }
}

}  // namespace ba
