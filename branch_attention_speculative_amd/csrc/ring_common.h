// Pieces shared by the bf16 matrix-core ring kernels: the ring walk over
// (step, chunk) segments, the swizzled LDS tile layout with its operand reads,
// and the direct global -> LDS tile loads.
#pragma once

#include "common.h"

namespace ba {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const void *gptr_t;
typedef __attribute__((address_space(3))) void *lptr_t;

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

// ---- LDS tile layout ------------------------------------------------------
// Tiles hold 64 rows x 128 bf16 columns, row-major with 256-byte rows (no
// padding). Bank conflicts are avoided by an XOR swizzle of the 16-byte
// chunks: logical chunk c of row r sits at physical chunk c ^ swz(r), with
// swz(r) = ((r & 3) << 2) | ((r >> 2) & 3). Measured on gfx950 with the
// SQ_LDS_BANK_CONFLICT counter, both access patterns below are conflict-free
// under it: 16 lanes reading one 16-byte chunk of 16 consecutive rows, and the
// transpose read (4 rows x 4 consecutive chunks per pair of 16-lane groups).
constexpr int kRS = 128;  // LDS row stride (bf16 elements)

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// element offset of (row, col) in a swizzled tile
__device__ __forceinline__ int toff(int r, int col) {
  return r * kRS + (((col >> 3) ^ swz(r)) << 3) + (col & 7);
}

// Natural operand from a tile X[row][col]: lane l takes row row0 + l%32 and
// the 8 columns col0 + 8*(l/32) .. +7 (col0 a multiple of 16). Serves A
// operands (rows = M, cols = K) and B operands (rows = N, cols = K).
__device__ __forceinline__ bf16x8 lds_nat(const u16 *X, int row0, int col0, int lane) {
  return as_bf16x8(
      *reinterpret_cast<const u32x4 *>(X + toff(row0 + (lane & 31), col0 + 8 * (lane >> 5))));
}

// Transposed operand from a tile X[k][m], for a contraction over the tile's
// rows: the operand element (m, slot s) is X[k0 + kslot16(s)][m0 + m]. Two
// ds_read_b64_tr_b16 per lane: inside each 16-lane group, lane j receives
// element j%4 of the 8-byte chunks addressed by lanes 4e + j/4 (e = 0..3), so
// pointing lane i at row (i/4) and column chunk (i%4) hands lane j four
// consecutive rows of column j.
__device__ __forceinline__ bf16x8 lds_tr(const u16 *X, int k0, int m0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int mb = (g & 1) << 4, h = g >> 1;
  const int r0 = k0 + 4 * h + (i >> 2);
  const int col = m0 + mb + 4 * (i & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(X + toff(r0, col)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(X + toff(r0 + 8, col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// Direct global -> LDS load of a 64-row x 128-col bf16 tile into the
// swizzled layout. global_load_lds_dwordx4 writes lane i's 16 bytes at the
// wave-uniform LDS base + 16 i, so each wave instruction fills 64 consecutive
// physical chunks (4 rows); lane i of instruction J fills row 4J + i/16,
// physical chunk i%16, i.e. logical chunk (i%16) ^ swz(row). The 16
// instructions of a tile are shared by the NW waves of the workgroup.
// rowaddr(row) gives the global address of a row's first element and must
// stay in bounds. Completion is tracked by vmcnt: dma_wait() before the
// barrier that publishes the tile.
template <int NW = 4, class RowAddr>
__device__ __forceinline__ void dma_tile64(u16 *lds_tile, RowAddr rowaddr, int wave, int lane) {
#pragma unroll
  for (int jj = 0; jj < 16 / NW; ++jj) {
    const int J = wave + NW * jj;
    const int row = 4 * J + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    const u16 *src = rowaddr(row) + 8 * c;
    __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(lds_tile + 512 * J), 16, 0, 0);
  }
}

// 64 consecutive 4-byte values (lane i -> element i) into LDS.
__device__ __forceinline__ void dma_dword64(void *lds_dst, const void *src_lane) {
  __builtin_amdgcn_global_load_lds((gptr_t)src_lane, (lptr_t)lds_dst, 4, 0, 0);
}

__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Value of lane 0, held in a scalar register (the argument must be uniform).
__device__ __forceinline__ int uniform_int(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Max / sum of a value over lanes l and l ^ 32 (v_permlane32_swap exchanges
// the upper half of one register with the lower half of the other; with the
// same value in both, each lane ends up with its partner's value in one of
// the two results and its own in the other).
__device__ __forceinline__ float xhalf_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over the bytes [base, base + bytes). Loads at offsets at or
// beyond `bytes` return zeros instead of touching memory, which is how the
// tile loads below stop at the end of a chunk or row range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
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

// ---- run list (the walk for short chunks) ----------------------------------
// The same walk as a list of runs built once per tile: the visible segments in
// walk order, where a shard's head and tail chunk of the sequence become one
// run of 2c keys when every row of the tile sees both in full (they are
// adjacent rows of the shard, and then no key of the run needs masking). The
// list lives in LDS and is walked by index, so the per-block walk logic is a
// few scalar loads instead of the segment arithmetic: on workloads with short
// chunks (hundreds of rows) that logic and the partial blocks at chunk ends
// weigh more than on long chunks.
constexpr int kMaxRuns = 128;  // 2 C segments, C <= 64

struct RunSeg {
  int n_hi, n_full, cpos0, pad;
  int64_t krow;
};

__device__ __forceinline__ Seg run_seg(int sg, const QTile &t, int C, int r, int n_local) {
  const int i = sg >> 1, half = sg & 1;
  int sh = r - i;
  if (sh < 0) sh += C;
  const int tail = 2 * C - 1 - sh;
  Seg s;
  s.krow = int64_t(sh) * n_local + t.seq_off + int64_t(half) * t.c;
  if (t.p_min >= (tail + 1) * t.c - 1) {
    // every row sees both chunks in full (no pad row in the tile, no pad key
    // in them): one run from the head chunk's first row; cpos0 is placed so
    // that bound - cpos0 >= 2c - 1 for every row, i.e. nothing is masked
    s.cpos0 = (tail - 1) * t.c;
    s.n_hi = s.n_full = half ? 0 : 2 * t.c;
    return s;
  }
  s.cpos0 = (half ? tail : sh) * t.c;
  s.n_hi = min(max(t.p_max - s.cpos0 + 1, 0), t.c);
  s.n_full = min(max(t.p_min - s.cpos0 + 1, 0), t.c);
  return s;
}

// Built by one wave: segment sg = 64 j + lane, the live ones (n_hi > 0)
// compacted in order with a ballot.
__device__ __forceinline__ void build_runs(RunSeg *runs, int *n_runs, const QTile &t, int C, int r,
                                           int n_local, int lane) {
  int base = 0;
  for (int sg0 = 0; sg0 < 2 * C; sg0 += 64) {
    const int sg = sg0 + lane;
    Seg s{0, 0, 0, 0};
    if (sg < 2 * C) s = run_seg(sg, t, C, r, n_local);
    const bool live = s.n_hi > 0;
    const uint64_t m = __ballot(live);
    const int at = base + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
    if (live) runs[at] = RunSeg{s.n_hi, s.n_full, s.cpos0, 0, s.krow};
    base += __popcll(m);
  }
  if (lane == 0) *n_runs = base;
}

__device__ __forceinline__ Seg load_run(const RunSeg *runs, int k) {
  const RunSeg v = runs[k];
  Seg s;
  s.n_hi = uniform_int(v.n_hi);
  s.n_full = uniform_int(v.n_full);
  s.cpos0 = uniform_int(v.cpos0);
  const uint64_t kr = uint64_t(v.krow);
  s.krow = int64_t((uint64_t(uint32_t(uniform_int(int(kr >> 32)))) << 32) |
                   uint32_t(uniform_int(int(kr & 0xffffffffu))));
  return s;
}

__device__ __forceinline__ void first_run(int &k, int &j0, Seg &s, const RunSeg *runs, int n_runs) {
  k = 0;
  j0 = 0;
  if (n_runs > 0) s = load_run(runs, 0);
}

template <int BN>
__device__ __forceinline__ void next_run(int &k, int &j0, Seg &s, const RunSeg *runs, int n_runs) {
  j0 += BN;
  if (j0 < s.n_hi) return;
  j0 = 0;
  if (++k < n_runs) s = load_run(runs, k);
}

// ---- precomputed per-lane offsets ----------------------------------------
// swz(r) only depends on r & 15, so shifting a tile row by a multiple of 16
// moves every address by a constant. The byte offsets below are computed
// once per kernel; the reads then add only compile-time immediates.

// lds_nat with row0 = 0: byte offset for each of the 8 column steps ks.
struct NatOff {
  int o[8];
};
__device__ __forceinline__ NatOff nat_offsets(int lane) {
  NatOff r;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) r.o[ks] = 2 * toff(lane & 31, 16 * ks + 8 * (lane >> 5));
  return r;
}
// natural operand: rows row0 + (lane & 31), columns 16 ks + 8 (lane / 32) ..
// (row0 a multiple of 16)
__device__ __forceinline__ bf16x8 lds_nat_o(const u16 *X, int row0, int ks, const NatOff &no) {
  return as_bf16x8(*reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(X) + no.o[ks] +
                                                    row0 * (2 * kRS)));
}

// lds_tr with k0 = 0: byte offsets of the two reads for each 32-column step dt.
struct TrOff {
  int o[2][4];
};
__device__ __forceinline__ TrOff tr_offsets(int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int mb = (g & 1) << 4, h = g >> 1;
  TrOff r;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      r.o[q][dt] = 2 * toff(4 * h + (i >> 2) + 8 * q, 32 * dt + mb + 4 * (i & 3));
  return r;
}
// transposed operand with rows k0 .. k0 + 15 (k0 a multiple of 16), columns
// 32 dt .. 32 dt + 31 (see lds_tr)
__device__ __forceinline__ bf16x8 lds_tr_o(const u16 *X, int k0, int dt, const TrOff &to) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const char *base = reinterpret_cast<const char *>(X) + k0 * (2 * kRS);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + to.o[0][dt]));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + to.o[1][dt]));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// Direct tile load of 64 rows whose addresses are base + rowoff(row): the
// per-lane part of the address is fixed for the kernel (DmaOff), only the
// wave-uniform base changes from tile to tile.
template <int NW>
struct DmaOff {
  uint32_t o[16 / NW];  // byte offsets from the tile base, one per instruction
};
// rowoff(row): element offset of tile row `row` from the tile base.
template <int NW, class RowOff>
__device__ __forceinline__ DmaOff<NW> dma_offsets(int wave, int lane, RowOff rowoff) {
  DmaOff<NW> r;
#pragma unroll
  for (int jj = 0; jj < 16 / NW; ++jj) {
    const int J = wave + NW * jj;
    const int row = 4 * J + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    r.o[jj] = uint32_t((int64_t(rowoff(row)) + 8 * c) * 2);
  }
  return r;
}
// Tile load through a buffer resource whose base is the tile's first row:
// no per-lane address arithmetic, and rows whose offset lies past the
// resource's extent are not read (zeros). `wave` must be uniform.
template <int NW>
__device__ __forceinline__ void dma_tile64_buf(u16 *lds_tile, __amdgpu_buffer_rsrc_t rs,
                                               const DmaOff<NW> &d, int wave) {
#pragma unroll
  for (int jj = 0; jj < 16 / NW; ++jj) {
    const int J = wave + NW * jj;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(lds_tile + 512 * J), 16, d.o[jj], 0, 0, 0);
  }
}

// Zero `n` u16 of LDS (n a multiple of 8 * nthreads), so that tile rows a
// load leaves out hold finite values.
__device__ __forceinline__ void lds_zero(u16 *p, int n, int tid, int nthreads) {
  for (int i = 8 * tid; i < n; i += 8 * nthreads) *reinterpret_cast<u32x4 *>(p + i) = u32x4{0, 0, 0, 0};
}

// ---- fp8 (OCP E4M3) operands -------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- fp8 K tile layout ------------------------------------------------------
// 64 key rows x 128 fp8 bytes, no padding; logical 16-byte chunk c of row r
// sits at physical chunk c ^ swz8(r), swz8(r) = (r >> 1) & 7. Rows are 128
// bytes (half the 256-byte bank sweep), so the 16 lanes of a quarter wave
// that read one chunk of 16 consecutive rows hit bank groups
// 8 (r & 1) + (c ^ swz8(r)): the even rows fill groups 0..7 and the odd rows
// 8..15, each exactly once.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// 32x32x64 fp8 (E4M3) x fp8 matrix-core product, fp32 accumulate. Operand
// lane layout (lane l, i = l % 32, h = l / 32): A (32 x 64): A[i][32h .. 32h+31];
// B (64 x 32): B[32h .. 32h+31][i]; C as for mfma32.
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Byte offsets of this lane's two 16-byte reads of the A operand for key
// rows 0..31 and D step kk (bytes 64 kk + 32 h .. + 31): add 32 * 128 for
// key rows 32..63.
struct Nat8Off {
  int o[2][2];
};
__device__ __forceinline__ Nat8Off nat8_offsets(int lane) {
  const int i = lane & 31, h = lane >> 5;
  Nat8Off r;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int t = 0; t < 2; ++t) r.o[kk][t] = 128 * i + 16 * ((4 * kk + 2 * h + t) ^ swz8(i));
  return r;
}
__device__ __forceinline__ i32x8 lds_nat8(const u16 *X, int row0, int kk, const Nat8Off &no) {
  const char *b = reinterpret_cast<const char *>(X) + 128 * row0;
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(b + no.o[kk][0]);
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(b + no.o[kk][1]);
  return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
               int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

// Direct global -> LDS load of a 64-row fp8 K tile: 8 KB, one 1 KB
// instruction per wave of the 8. Instruction J fills rows 8J .. 8J + 7; its
// lane i writes physical chunk i % 8 of row 8J + i / 8, i.e. logical chunk
// (i % 8) ^ swz8(row). rowstride: bytes between key rows in global memory.
__device__ __forceinline__ uint32_t dma8_offset(int wave, int lane, int64_t rowstride) {
  const int row = 8 * wave + (lane >> 3);
  const int c = (lane & 7) ^ swz8(row);
  return uint32_t(int64_t(row) * rowstride + 16 * c);
}
__device__ __forceinline__ void dma_tile64_f8(u16 *lds_tile, __amdgpu_buffer_rsrc_t rs,
                                              uint32_t off, int wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(reinterpret_cast<char *>(lds_tile) + 1024 * wave),
                                           16, off, 0, 0, 0);
}

}  // namespace ba
