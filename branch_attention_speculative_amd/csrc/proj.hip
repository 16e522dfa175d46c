// The draft layer's projection of hidden states to the attention inputs:
// q, k, v = x W^T split into heads, a per-head RMS norm of q and k, and
// rotary position embedding at each row's position (bf16 in, fp32
// accumulate, d = 128).
//
// This is the step before branch attention in the draft forward (rainbus
// analysis, method steps, step four: EAGLE-3 runs its training-time-test
// passes, DFlash produces a whole block, DSpark adds a Markov head; paperlens
// walkthrough, "The two walls": a TTT branch grows from every position). It
// writes straight into the attention's layouts: main rows into q and this
// rank's K/V shard, branch rows into qb/kb/vb at their anchor's slots. A
// TTT pass j takes the step-major hidden states of step j (one row per local
// anchor) and fills branch row j of every anchor.
//
// One workgroup (4 waves) computes one head (128 output dims) for 128 rows:
// Y^T = W_h X^T, the dims as the MFMA M side, so in the output registers a
// lane holds one row and half of that row's 128 dims (the other half in lane
// l ^ 32). The head's RMS norm is then one exchange between the two lanes,
// and RoPE's dim pairs (i, i + 64) sit in the same lane. W and X stream
// through LDS in 64-wide steps of the hidden dimension (double-buffered,
// direct global -> LDS loads into 128-byte rows swizzled against bank
// conflicts, as the fp8 K tiles of the forward).

#include "kernels.h"
#include "ring_common.h"

namespace ba {

namespace {

constexpr int kPR = 128;    // rows per tile
constexpr int kPK = 64;     // hidden elements per step
constexpr int kPWaves = 4;  // waves per workgroup (32 rows each)

// 128-byte LDS rows: logical 16-byte chunk c of row r at c ^ ((r >> 1) & 7)
__device__ __forceinline__ int pswz(int r) { return (r >> 1) & 7; }

// byte offset of this lane's MFMA operand (row r0 + lane % 32, elements
// 16 ks + 8 (lane / 32) .. + 7 of the step) in a 128-byte-row tile; r0 is a
// multiple of 16, so the swizzle only depends on the lane
__device__ __forceinline__ int op_off(int r0, int ks, int lane) {
  const int i = lane & 31, h = lane >> 5;
  return (r0 + i) * 128 + 16 * ((2 * ks + h) ^ pswz(i));
}

// The 16 one-kilobyte load instructions of a 128 x 64 bf16 tile, four per
// wave: instruction J fills rows 8J .. 8J + 7; lane i writes physical chunk
// i % 8 of row 8J + i / 8, i.e. loads logical chunk (i % 8) ^ pswz(row).
// rowbytes: bytes between rows in global memory.
struct TileOff {
  uint32_t o[4];
};
__device__ __forceinline__ TileOff tile_offsets(int wave, int lane, uint32_t rowbytes) {
  TileOff t;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int J = wave + kPWaves * jj;
    const int row = 8 * J + (lane >> 3);
    t.o[jj] = uint32_t(row) * rowbytes + 16u * uint32_t((lane & 7) ^ pswz(row));
  }
  return t;
}
// soff: byte offset of the step inside each row (wave-uniform)
__device__ __forceinline__ void load_tile(u16 *lds, __amdgpu_buffer_rsrc_t rs, const TileOff &t,
                                          int wave, uint32_t soff) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int J = wave + kPWaves * jj;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(reinterpret_cast<char *>(lds) + 1024 * J),
                                             16, t.o[jj], soff, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 lds_op(const u16 *tile, int off) {
  return as_bf16x8(*reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(tile) + off));
}

__global__ __launch_bounds__(kPWaves * 64) void qkv_project_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sW0[kPR * kPK];
  __shared__ __attribute__((aligned(16))) u16 sX0[kPR * kPK];
  __shared__ __attribute__((aligned(16))) u16 sW1[kPR * kPK];
  __shared__ __attribute__((aligned(16))) u16 sX1[kPR * kPK];

  const int nheads = a.hq + 2 * a.hkv;
  const int head = blockIdx.x % nheads;
  const int row0 = (blockIdx.x / nheads) * kPR;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform_int(tid >> 6);
  const int nrows = min(kPR, a.nrows - row0);
  const uint32_t rowbytes = uint32_t(a.hidden) * 2;
  // W rows of this head and X rows of this tile; rows past the tile's end are
  // outside the X resource and load as zeros
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(static_cast<const u16 *>(a.w) + int64_t(head) * 128 * a.hidden,
                                             uint32_t(128) * rowbytes);
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(static_cast<const u16 *>(a.x) + int64_t(row0) * a.hidden,
                                             uint32_t(nrows) * rowbytes);
  const TileOff to = tile_offsets(wave, lane, rowbytes);

  f32x16 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
  int aoff[4][4], boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) aoff[mt][ks] = op_off(32 * mt, ks, lane);
    boff[ks] = op_off(32 * wave, ks, lane);
  }

  const int nsteps = a.hidden / kPK;
  load_tile(sW0, rw, to, wave, 0);
  load_tile(sX0, rx, to, wave, 0);
  dma_wait();
  __syncthreads();
  auto step = [&](const u16 *W, const u16 *X, u16 *Wn, u16 *Xn, int s) {
    if (s + 1 < nsteps) {
      load_tile(Wn, rw, to, wave, uint32_t(s + 1) * kPK * 2);
      load_tile(Xn, rx, to, wave, uint32_t(s + 1) * kPK * 2);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = lds_op(X, boff[ks]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma32(lds_op(W, aoff[mt][ks]), b, acc[mt]);
    }
    dma_wait();
    __syncthreads();
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(sW0, sX0, sW1, sX1, s);
    if (s + 1 < nsteps) step(sW1, sX1, sW0, sX0, s + 1);
  }

  // ---- epilogue: this lane's row and its 64 dims 32 mt + 8 g + 4 h + e ----
  const int i = lane & 31, h = lane >> 5;
  const int rl = 32 * wave + i;
  if (rl >= nrows) return;
  const int r = row0 + rl;  // input row
  // output row and position
  int orow, pos;
  bool zero = false;
  if (a.target == 0) {
    orow = r;
    pos = a.bound_main[r];
    zero = pos < 0;  // pad row
  } else if (a.step >= 0) {
    orow = a.branch_off[r] + a.step;
    pos = a.anchor_pos[r] + 1 + a.step;
  } else {
    orow = r;
    const int an = a.b_anchor[r];
    pos = a.anchor_pos[an] + 1 + (r - a.branch_off[an]);
  }
  const bool is_q = head < a.hq, is_k = !is_q && head < a.hq + a.hkv;
  const u16 *nw = static_cast<const u16 *>(is_q ? a.q_norm : a.k_norm);
  if ((is_q || is_k) && nw != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) ss = fmaf(acc[mt][v], acc[mt][v], ss);
    const float rms = rsqrtf(xhalf_sum(ss) * (1.f / 128.f) + a.eps);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w2 = *reinterpret_cast<const u32x2 *>(nw + 32 * mt + 8 * g + 4 * h);
        const float wv[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xffff0000u),
                             __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][4 * g + e] *= rms * wv[e];
      }
  }
  if ((is_q || is_k) && a.rope) {
    // (x_j, x_{j+64}) turns by pos * theta^(-2j/128); the angle is reduced
    // modulo 2 pi in double precision, so large positions keep their phase
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
        const double ang = double(pos) * a.inv_freq[j];
        const double turns = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
        const float red = float(fma(-turns, 6.283185307179586, ang));
        float sn, cs;
        sincosf(red, &sn, &cs);
        const float x1 = acc[mt][v], x2 = acc[mt + 2][v];
        acc[mt][v] = x1 * cs - x2 * sn;
        acc[mt + 2][v] = x2 * cs + x1 * sn;
      }
  }
  u16 *out;
  int64_t base;
  if (is_q) {
    out = static_cast<u16 *>(a.q);
    base = (int64_t(orow) * a.hq + head) * 128;
  } else if (is_k) {
    out = static_cast<u16 *>(a.k);
    base = (int64_t(orow) * a.hkv + (head - a.hq)) * 128;
  } else {
    out = static_cast<u16 *>(a.v);
    base = (int64_t(orow) * a.hkv + (head - a.hq - a.hkv)) * 128;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w.x = zero ? 0u : cvt_pk_bf16(acc[mt][4 * g + 0], acc[mt][4 * g + 1]);
      w.y = zero ? 0u : cvt_pk_bf16(acc[mt][4 * g + 2], acc[mt][4 * g + 3]);
      *reinterpret_cast<u32x2 *>(out + base + 32 * mt + 8 * g + 4 * h) = w;
    }
}

}  // namespace

hipError_t launch_qkv_project(const ProjArgs &a, hipStream_t s) {
  const int64_t tiles = (int64_t(a.nrows) + kPR - 1) / kPR;
  const int64_t blocks = tiles * (a.hq + 2 * a.hkv);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_project_kernel, dim3(uint32_t(blocks)), dim3(kPWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
