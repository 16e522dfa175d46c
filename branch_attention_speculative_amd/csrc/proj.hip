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
// One workgroup (4 waves) computes one head (128 output dims) for 256 rows:
// Y^T = W_h X^T, the dims as the MFMA M side, so in the output registers a
// lane holds one row and half of that row's 128 dims (the other half in lane
// l ^ 32). The head's RMS norm is then one exchange between the two lanes,
// and RoPE's dim pairs (i, i + 64) sit in the same lane. The hidden dimension
// streams in steps of 64. W, which all four waves use, goes through LDS
// (double-buffered, direct global -> LDS loads into 128-byte rows swizzled
// against bank conflicts); each wave's 64 X rows are its own and go straight
// into registers one step ahead. Inside a step the contraction order is
// permuted so that a lane's X operand is one contiguous 64-byte piece of its
// row: lane half h takes hidden elements 32 h .. 32 h + 31 of the step,
// product ks of them 32 h + 8 ks .. + 7, and the W operand read from LDS
// follows the same order.

#include "kernels.h"
#include "ring_common.h"

namespace ba {

namespace {

constexpr int kPR = 256;    // rows per tile
constexpr int kPW = 128;    // W rows (output dims) per tile: one head
constexpr int kPK = 64;     // hidden elements per step
constexpr int kPWaves = 4;  // waves per workgroup (64 rows each)

// 128-byte LDS rows: logical 16-byte chunk c of row r at c ^ ((r >> 1) & 7)
__device__ __forceinline__ int pswz(int r) { return (r >> 1) & 7; }

// The 16 one-kilobyte load instructions of the 128 x 64 W tile, four per
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
__device__ __forceinline__ void load_w(u16 *lds, __amdgpu_buffer_rsrc_t rs, const TileOff &t, int wave,
                                       uint32_t soff) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int J = wave + kPWaves * jj;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(reinterpret_cast<char *>(lds) + 1024 * J),
                                             16, t.o[jj], soff, 0, 0);
  }
}

// this lane's X operands of one step: rows 64 wave + 32 nt + lane % 32,
// 16 bytes per product ks (rows past the tile's end are outside the
// resource and load as zeros)
struct XOps {
  u32x4 v[2][4];
};
__device__ __forceinline__ void load_x(XOps &x, __amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[2],
                                       uint32_t soff) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, off[nt] + 16u * ks, soff, 0);
      x.v[nt][ks] = u32x4{r[0], r[1], r[2], r[3]};
    }
}

__device__ __forceinline__ bf16x8 lds_op(const u16 *tile, int off) {
  return as_bf16x8(*reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(tile) + off));
}

__global__ __launch_bounds__(kPWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_project_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sW0[kPW * kPK];
  __shared__ __attribute__((aligned(16))) u16 sW1[kPW * kPK];

  const int nheads = a.hq + 2 * a.hkv;
  const int head = blockIdx.x % nheads;
  const int row0 = (blockIdx.x / nheads) * kPR;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform_int(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int nrows = min(kPR, a.nrows - row0);
  const uint32_t rowbytes = uint32_t(a.hidden) * 2;
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(static_cast<const u16 *>(a.w) + int64_t(head) * kPW * a.hidden,
                                             uint32_t(kPW) * rowbytes);
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(static_cast<const u16 *>(a.x) + int64_t(row0) * a.hidden,
                                             uint32_t(nrows) * rowbytes);
  const TileOff tw = tile_offsets(wave, lane, rowbytes);
  uint32_t xoff[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) xoff[nt] = uint32_t(64 * wave + 32 * nt + i) * rowbytes + 64u * h;
  // W operand of dim tile mt, product ks: row 32 mt + i, logical chunk 4 h + ks
  int aoff[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) aoff[mt][ks] = (32 * mt + i) * 128 + 16 * ((4 * h + ks) ^ pswz(i));

  // acc[nt][mt]: rows 64 wave + 32 nt + i, dims 32 mt + 8 g + 4 h + e
  f32x16 acc[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = f32x16{};

  const int nsteps = a.hidden / kPK;
  XOps xc, xn;
  load_w(sW0, rw, tw, wave, 0);
  load_x(xc, rx, xoff, 0);
  dma_wait();
  __syncthreads();
  auto step = [&](const u16 *W, u16 *Wn, int s) {
    if (s + 1 < nsteps) {
      load_w(Wn, rw, tw, wave, uint32_t(s + 1) * kPK * 2);
      load_x(xn, rx, xoff, uint32_t(s + 1) * kPK * 2);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b0 = as_bf16x8(xc.v[0][ks]), b1 = as_bf16x8(xc.v[1][ks]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 w = lds_op(W, aoff[mt][ks]);
        acc[0][mt] = mfma32(w, b0, acc[0][mt]);
        acc[1][mt] = mfma32(w, b1, acc[1][mt]);
      }
    }
    dma_wait();
    __syncthreads();
    xc = xn;
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(sW0, sW1, s);
    if (s + 1 < nsteps) step(sW1, sW0, s + 1);
  }

  // ---- epilogue: per row sub-tile, this lane's row and its 64 dims
  // 32 mt + 8 g + 4 h + e ----
  const bool is_q = head < a.hq, is_k = !is_q && head < a.hq + a.hkv;
  const u16 *nw = static_cast<const u16 *>(is_q ? a.q_norm : a.k_norm);
  auto epilogue = [&](f32x16 (&y)[4], int nt) {
    const int rl = 64 * wave + 32 * nt + i;
    // both lanes of a row (l and l ^ 32) take the same branch, which the
    // lane-pair exchange of the norm relies on
    if (rl >= nrows) return;
    const int r = row0 + rl;  // input row
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
    if ((is_q || is_k) && nw != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) ss = fmaf(y[mt][v], y[mt][v], ss);
      const float rms = rsqrtf(xhalf_sum(ss) * (1.f / 128.f) + a.eps);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w2 = *reinterpret_cast<const u32x2 *>(nw + 32 * mt + 8 * g + 4 * h);
          const float wv[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xffff0000u),
                               __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xffff0000u)};
#pragma unroll
          for (int e = 0; e < 4; ++e) y[mt][4 * g + e] *= rms * wv[e];
        }
    }
    if ((is_q || is_k) && a.rope) {
      // (x_j, x_{j+64}) turns by pos * theta^(-2j/128) radians. The angle is
      // taken in revolutions and reduced to [-1/2, 1/2] in double precision,
      // so large positions keep their phase, and the hardware sine and cosine
      // (which take revolutions) finish it in single precision.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
          const double rev = double(pos) * a.inv_freq[j] * 0.15915494309189535;  // 1 / (2 pi)
          const float red = float(rev - rint(rev));
          const float sn = __builtin_amdgcn_sinf(red), cs = __builtin_amdgcn_cosf(red);
          const float x1 = y[mt][v], x2 = y[mt + 2][v];
          y[mt][v] = x1 * cs - x2 * sn;
          y[mt + 2][v] = x2 * cs + x1 * sn;
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
        w.x = zero ? 0u : cvt_pk_bf16(y[mt][4 * g + 0], y[mt][4 * g + 1]);
        w.y = zero ? 0u : cvt_pk_bf16(y[mt][4 * g + 2], y[mt][4 * g + 3]);
        *reinterpret_cast<u32x2 *>(out + base + 32 * mt + 8 * g + 4 * h) = w;
      }
  };
  epilogue(acc[0], 0);
  epilogue(acc[1], 1);
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
