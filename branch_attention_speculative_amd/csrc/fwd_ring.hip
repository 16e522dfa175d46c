// Ring-step causal partial, forward (bf16 in, fp32 accumulate, D = 128).
//
// One workgroup owns a query tile: up to 128 query vectors (consecutive rows
// of one sequence chunk x the G q-heads of one kv-head). It walks the virtual
// ring i = 0..C-1 over shard (r - i) mod C -- the K/V that would circulate
// while the queries stay (ai.info summary, Methodology; rainbus analysis,
// method steps, step two) -- and inside each shard the sequence's head chunk,
// then its tail chunk, in blocks of 64 keys. The online-softmax state
// (running max, sum, unnormalised O) is carried in registers across blocks
// and ring steps, which is the log-sum-exp merge between ring steps (rainbus
// analysis, core method, Eq. 2, applied incrementally). Key blocks past a
// tile's largest causal bound are never visited; blocks wholly inside its
// smallest bound skip the mask.
//
// Per wave: 32 query vectors. Scores are formed transposed, S^T = K Q^T, so a
// lane owns one query: the row max and sum need one cross-half exchange and
// the O rescale is a scalar per lane. O^T += V^T P^T takes P^T straight from
// the score registers; V is staged transposed in LDS with the kslot16 key
// order so that both operands agree.

#include "common.h"
#include "kernels.h"

namespace ba {

namespace {

constexpr int kBN = 64;        // keys per block
constexpr int kKStride = 136;  // LDS row stride (bf16) of [key][d] tiles: 128 + 8
constexpr int kTStride = 72;   // LDS row stride (bf16) of [d][key slot] tiles: 64 + 8

struct Seg {
  int n_hi;     // keys of this chunk visible to the tile's largest bound
  int n_full;   // keys visible to every row of the tile
  int cpos0;    // sequence position of the chunk's first key
  int64_t krow; // row of the chunk's first key in the [C * N] key array
};

// Segment sg = 2*i + half: ring step i (shard (r - i) mod C), head (0) or
// tail (1) chunk of the tile's sequence inside that shard.
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

// Advance to the next non-empty block: (sg, j0) -> next, sg == 2C when done.
__device__ __forceinline__ void next_block(int &sg, int &j0, Seg &s, const QTile &t, int C, int r,
                                           int n_local) {
  j0 += kBN;
  if (j0 < s.n_hi) return;
  j0 = 0;
  for (++sg; sg < 2 * C; ++sg) {
    s = seg_info(sg, t, C, r, n_local);
    if (s.n_hi > 0) return;
  }
}

__device__ __forceinline__ void first_block(int &sg, int &j0, Seg &s, const QTile &t, int C, int r,
                                            int n_local) {
  j0 = 0;
  for (sg = 0; sg < 2 * C; ++sg) {
    s = seg_info(sg, t, C, r, n_local);
    if (s.n_hi > 0) return;
  }
}

struct KVRegs {
  u32x4 k[4];  // natural K: 4 x 16 B per thread
  u32x2 v[8];  // V for the transposed store: 8 keys x 4 d per thread
};

__device__ __forceinline__ void load_kv(KVRegs &R, const u16 *__restrict__ K,
                                        const u16 *__restrict__ V, const Seg &s, int j0, int g,
                                        int hkv, int tid) {
  const int64_t rs = int64_t(hkv) * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int key = id >> 4, dc = id & 15;
    const int kk = min(j0 + key, s.n_hi - 1);
    R.k[i] = *reinterpret_cast<const u32x4 *>(K + (s.krow + kk) * rs + g * 128 + dc * 8);
  }
  const int dgrp = tid & 31, kgrp = tid >> 5;
  const int u = kgrp >> 1, sub = kgrp & 1;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int key = 16 * u + kslot16(8 * sub + jj);
    const int kk = min(j0 + key, s.n_hi - 1);
    R.v[jj] = *reinterpret_cast<const u32x2 *>(V + (s.krow + kk) * rs + g * 128 + 4 * dgrp);
  }
}

__device__ __forceinline__ void store_kv(const KVRegs &R, u16 *sK, u16 *sVt, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int key = id >> 4, dc = id & 15;
    *reinterpret_cast<u32x4 *>(sK + key * kKStride + dc * 8) = R.k[i];
  }
  const int dgrp = tid & 31, kgrp = tid >> 5;
  const int u = kgrp >> 1, sub = kgrp & 1;
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    u32x4 w;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = (dd < 2) ? R.v[2 * p].x : R.v[2 * p].y;
      const uint32_t b = (dd < 2) ? R.v[2 * p + 1].x : R.v[2 * p + 1].y;
      w[p] = (dd & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<u32x4 *>(sVt + (4 * dgrp + dd) * kTStride + 16 * u + 8 * sub) = w;
  }
}

__global__ __launch_bounds__(256) void fwd_ring_bf16_kernel(FwdRingArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sK[kBN * kKStride];
  __shared__ __attribute__((aligned(16))) u16 sVt[128 * kTStride];

  const QTile t = a.qtiles[blockIdx.x];
  if (t.nrows == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hf = lane >> 5;
  const int m = wave * 32 + qi;
  const int rl = m >> a.log2G, hh = m & (a.G - 1);
  const bool valid = rl < t.nrows;
  const bool wave_active = (wave * 32) < (t.nrows << a.log2G);
  const int row = t.row0 + (valid ? rl : 0);
  const int h = t.g * a.G + hh;
  const u16 *Q = static_cast<const u16 *>(t.src ? a.qb : a.q);
  const u16 *K = static_cast<const u16 *>(a.k);
  const u16 *V = static_cast<const u16 *>(a.v);
  const int bound = valid ? (t.src ? a.bound_branch[row] : a.bound_main[row]) : -1;

  bf16x8 qreg[8];
  {
    const u16 *qp = Q + (int64_t(row) * a.hq + h) * 128 + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = valid ? *reinterpret_cast<const u32x4 *>(qp + ks * 16) : u32x4{0, 0, 0, 0};
      qreg[ks] = as_bf16x8(x);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  float mrun = kNegInf, lsum = 0.f;
  const float sl2 = a.scale_log2;

  int sg, j0;
  Seg s;
  first_block(sg, j0, s, t, a.C, a.r, a.n_local);
  KVRegs R;
  if (sg < 2 * a.C) load_kv(R, K, V, s, j0, t.g, a.hkv, tid);

  while (sg < 2 * a.C) {
    const Seg cs = s;
    const int cj0 = j0;
    next_block(sg, j0, s, t, a.C, a.r, a.n_local);
    __syncthreads();  // previous block's LDS reads are done
    store_kv(R, sK, sVt, tid);
    __syncthreads();
    if (sg < 2 * a.C) load_kv(R, K, V, s, j0, t.g, a.hkv, tid);  // prefetch, overlaps compute
    if (!wave_active) continue;

    // S^T = K Q^T for 64 keys (two 32-key tiles)
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a0 =
          as_bf16x8(*reinterpret_cast<const u32x4 *>(sK + qi * kKStride + ks * 16 + hf * 8));
      const bf16x8 a1 =
          as_bf16x8(*reinterpret_cast<const u32x4 *>(sK + (32 + qi) * kKStride + ks * 16 + hf * 8));
      s0 = mfma32(a0, qreg[ks], s0);
      s1 = mfma32(a1, qreg[ks], s1);
    }
    float x[32];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = s0[v] * sl2;
      x[16 + v] = s1[v] * sl2;
    }
    if (cj0 + kBN > cs.n_full) {
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int jj = cj0 + 32 * (v >> 4) + 8 * ((v & 15) >> 2) + 4 * hf + (v & 3);
        const bool vis = (jj < cs.n_hi) && (cs.cpos0 + jj <= bound);
        x[v] = vis ? x[v] : kNegInf;
      }
    }
    float bmax = x[0];
#pragma unroll
    for (int v = 1; v < 32; ++v) bmax = fmaxf(bmax, x[v]);
    bmax = fmaxf(bmax, wave_shfl_xor32(bmax));
    const float mnew = fmaxf(mrun, bmax);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(mrun - muse);
    mrun = mnew;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 32; ++v) {
      x[v] = fast_exp2(x[v] - muse);
      psum += x[v];
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    bf16x8 pb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 w;
#pragma unroll
      for (int p = 0; p < 4; ++p) w[p] = pack_bf2(x[8 * u + 2 * p], x[8 * u + 2 * p + 1]);
      pb[u] = as_bf16x8(w);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 av = as_bf16x8(
            *reinterpret_cast<const u32x4 *>(sVt + (32 * dt + qi) * kTStride + 16 * u + 8 * hf));
        acc[dt] = mfma32(av, pb[u], acc[dt]);
      }
    }
  }

  if (!valid) return;
  const float ltot = lsum + wave_shfl_xor32(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse = ltot > 0.f ? (mrun + log2f(ltot)) * kLn2 : kNegInf;
  const int64_t ob = (int64_t(row) * a.hq + h) * 128;
  if (t.src == 0) {
    u16 *O = static_cast<u16 *>(a.o);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * hf;
        u32x2 w;
        w.x = pack_bf2(acc[dt][4 * a4 + 0] * inv, acc[dt][4 * a4 + 1] * inv);
        w.y = pack_bf2(acc[dt][4 * a4 + 2] * inv, acc[dt][4 * a4 + 3] * inv);
        *reinterpret_cast<u32x2 *>(O + ob + d0) = w;
      }
    if (hf == 0) a.lse[int64_t(row) * a.hq + h] = lse;
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * hf;
        f32x4 w = {acc[dt][4 * a4 + 0] * inv, acc[dt][4 * a4 + 1] * inv,
                   acc[dt][4 * a4 + 2] * inv, acc[dt][4 * a4 + 3] * inv};
        *reinterpret_cast<f32x4 *>(a.om + ob + d0) = w;
      }
    if (hf == 0) a.lm[int64_t(row) * a.hq + h] = lse;
  }
}

}  // namespace

hipError_t launch_fwd_ring_bf16(const FwdRingArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_ring_bf16_kernel, dim3(n_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
