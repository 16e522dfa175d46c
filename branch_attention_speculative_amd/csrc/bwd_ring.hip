// Ring replay for the backward (bf16 in, fp32 accumulate, D = 128).
//
// The backward recomputes P = exp(s - LSE) from the merged LSE of the forward
// and replays the same virtual ring (rainbus analysis of arXiv:2609.07108,
// method steps, step five: the backward replays the ring and accumulates the
// gradients locally):
//   dP = dO V^T, dS = P (dP - Delta), dQ = scale dS K, dK = scale dS^T Q,
//   dV = P^T dO.
// Two kernels avoid atomics: a query-stationary one for dQ (same tiles and
// ring walk as the forward) and a key-stationary one for dK/dV, whose key
// tiles each see a suffix of the sequence's main rows and of its branch rows
// (query rows and anchors are stored in increasing position order, so the
// rows whose causal bound reaches a key form a suffix).

#include "common.h"
#include "kernels.h"

namespace ba {

namespace {

constexpr int kBN = 64;  // keys per block in the dQ kernel

struct Seg {
  int n_hi, n_full, cpos0;
  int64_t krow;
};

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

// ---------------------------------------------------------------------------
// dQ: query-stationary ring replay

struct DqRegs {
  u32x4 k[4], v[4];  // natural K and V rows: 4 x 16 B each per thread
  u32x2 kt[8];       // K for the transposed store: 8 keys x 4 d
};

__device__ __forceinline__ void dq_load(DqRegs &R, const u16 *__restrict__ K,
                                        const u16 *__restrict__ V, const Seg &s, int j0, int g,
                                        int hkv, int tid) {
  const int64_t rs = int64_t(hkv) * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int key = id >> 4, dc = id & 15;
    const int64_t off = (s.krow + min(j0 + key, s.n_hi - 1)) * rs + g * 128 + dc * 8;
    R.k[i] = *reinterpret_cast<const u32x4 *>(K + off);
    R.v[i] = *reinterpret_cast<const u32x4 *>(V + off);
  }
  const int dgrp = tid & 31, kgrp = tid >> 5;
  const int u = kgrp >> 1, sub = kgrp & 1;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int key = 16 * u + kslot16(8 * sub + jj);
    R.kt[jj] = *reinterpret_cast<const u32x2 *>(K + (s.krow + min(j0 + key, s.n_hi - 1)) * rs +
                                                 g * 128 + 4 * dgrp);
  }
}

__device__ __forceinline__ void dq_store(const DqRegs &R, u16 *sK, u16 *sV, u16 *sKt, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int key = id >> 4, dc = id & 15;
    *reinterpret_cast<u32x4 *>(sK + key * kNatStride + dc * 8) = R.k[i];
    *reinterpret_cast<u32x4 *>(sV + key * kNatStride + dc * 8) = R.v[i];
  }
  const int dgrp = tid & 31, kgrp = tid >> 5;
  const int u = kgrp >> 1, sub = kgrp & 1;
  store_t8x4(R.kt, sKt + (4 * dgrp) * kTrStride + 16 * u + 8 * sub, kTrStride);
}

__global__ __launch_bounds__(256) void bwd_dq_bf16_kernel(BwdDqArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sK[kBN * kNatStride];
  __shared__ __attribute__((aligned(16))) u16 sV[kBN * kNatStride];
  __shared__ __attribute__((aligned(16))) u16 sKt[128 * kTrStride];

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
  const u16 *DO = static_cast<const u16 *>(t.src ? a.doutb : a.dout);
  const u16 *K = static_cast<const u16 *>(a.k);
  const u16 *V = static_cast<const u16 *>(a.v);
  const int bound = valid ? (t.src ? a.bound_branch[row] : a.bound_main[row]) : -1;
  const int64_t qh = int64_t(row) * a.hq + h;
  const float lse = valid ? (t.src ? a.lseb[qh] : a.lse[qh]) : 0.f;
  const float lse2 = (bound >= 0) ? lse * kLog2e : 0.f;
  const float delta = (bound >= 0) ? a.delta[(t.src ? int64_t(a.n_local) * a.hq : 0) + qh] : 0.f;

  bf16x8 qreg[8], dreg[8];
  {
    const u16 *qp = Q + qh * 128 + hf * 8;
    const u16 *dp = DO + qh * 128 + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qreg[ks] = as_bf16x8(valid ? *reinterpret_cast<const u32x4 *>(qp + ks * 16) : u32x4{0, 0, 0, 0});
      dreg[ks] = as_bf16x8(valid ? *reinterpret_cast<const u32x4 *>(dp + ks * 16) : u32x4{0, 0, 0, 0});
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  const float sl2 = a.scale_log2;

  int sg, j0;
  Seg s;
  first_block(sg, j0, s, t, a.C, a.r, a.n_local);
  DqRegs R;
  if (sg < 2 * a.C) dq_load(R, K, V, s, j0, t.g, a.hkv, tid);

  while (sg < 2 * a.C) {
    const Seg cs = s;
    const int cj0 = j0;
    next_block(sg, j0, s, t, a.C, a.r, a.n_local);
    __syncthreads();
    dq_store(R, sK, sV, sKt, tid);
    __syncthreads();
    if (sg < 2 * a.C) dq_load(R, K, V, s, j0, t.g, a.hkv, tid);
    if (!wave_active) continue;

    // S^T = K Q^T and dP^T = V dO^T for 64 keys
    f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int o0 = qi * kNatStride + ks * 16 + hf * 8;
      const int o1 = (32 + qi) * kNatStride + ks * 16 + hf * 8;
      s0 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sK + o0)), qreg[ks], s0);
      s1 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sK + o1)), qreg[ks], s1);
      p0 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sV + o0)), dreg[ks], p0);
      p1 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sV + o1)), dreg[ks], p1);
    }
    const bool need_mask = cj0 + kBN > cs.n_full;
    float ds[32];
#pragma unroll
    for (int v = 0; v < 32; ++v) {
      const float sv = v < 16 ? s0[v] : s1[v - 16];
      const float dpv = v < 16 ? p0[v] : p1[v - 16];
      float p = fast_exp2(sv * sl2 - lse2);
      if (need_mask) {
        const int jj = cj0 + 32 * (v >> 4) + 8 * ((v & 15) >> 2) + 4 * hf + (v & 3);
        const bool vis = (jj < cs.n_hi) && (cs.cpos0 + jj <= bound);
        p = vis ? p : 0.f;
      }
      ds[v] = p * (dpv - delta);
    }
    bf16x8 db[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 w;
#pragma unroll
      for (int p = 0; p < 4; ++p) w[p] = pack_bf2(ds[8 * u + 2 * p], ds[8 * u + 2 * p + 1]);
      db[u] = as_bf16x8(w);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 ak = as_bf16x8(
            *reinterpret_cast<const u32x4 *>(sKt + (32 * dt + qi) * kTrStride + 16 * u + 8 * hf));
        acc[dt] = mfma32(ak, db[u], acc[dt]);
      }
  }

  if (!valid) return;
  const float sc = a.scale;
  u16 *DQ = static_cast<u16 *>(t.src ? a.dqb : a.dq);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d0 = 32 * dt + 8 * a4 + 4 * hf;
      float x0 = acc[dt][4 * a4 + 0] * sc, x1 = acc[dt][4 * a4 + 1] * sc;
      float x2 = acc[dt][4 * a4 + 2] * sc, x3 = acc[dt][4 * a4 + 3] * sc;
      if (t.src) {
        const f32x4 l = *reinterpret_cast<const f32x4 *>(a.dq_local + qh * 128 + d0);
        x0 += l[0];
        x1 += l[1];
        x2 += l[2];
        x3 += l[3];
      }
      u32x2 w;
      w.x = pack_bf2(x0, x1);
      w.y = pack_bf2(x2, x3);
      *reinterpret_cast<u32x2 *>(DQ + qh * 128 + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// dK / dV: key-stationary ring replay

constexpr int kQB = 64;  // query vectors per inner block

__global__ __launch_bounds__(256) void bwd_dkdv_bf16_kernel(BwdDkdvArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sQ[kQB * kNatStride];
  __shared__ __attribute__((aligned(16))) u16 sD[kQB * kNatStride];
  __shared__ __attribute__((aligned(16))) u16 sQt[128 * kTrStride];
  __shared__ __attribute__((aligned(16))) u16 sDt[128 * kTrStride];
  __shared__ __attribute__((aligned(16))) float sL[kQB];
  __shared__ __attribute__((aligned(16))) float sDel[kQB];
  __shared__ __attribute__((aligned(16))) int sB[kQB];

  const KTile t = a.ktiles[blockIdx.x];
  if (t.nkeys == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hf = lane >> 5;
  const int kk = wave * 32 + qi;  // this lane's key inside the tile
  const bool kvalid = kk < t.nkeys;
  const int kpos = t.kpos0 + kk;
  const int G = a.G, log2G = a.log2G;
  const int64_t krow = int64_t(t.shard) * a.n_local + t.krow0 + min(kk, t.nkeys - 1);
  const int64_t koff = (krow * a.hkv + t.g) * 128;
  const u16 *K = static_cast<const u16 *>(a.k);
  const u16 *V = static_cast<const u16 *>(a.v);

  bf16x8 kreg[8], vreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(K + koff + ks * 16 + hf * 8));
    vreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(V + koff + ks * 16 + hf * 8));
  }
  f32x16 adk[4], adv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    adk[dt] = f32x16{};
    adv[dt] = f32x16{};
  }
  const float sl2 = a.scale_log2;
  const int RB = kQB >> log2G;  // rows per inner block
  const bool wave_active = (wave * 32) < t.nkeys;

  for (int src = 0; src < 2; ++src) {
    const int lo = src ? t.qb_start : t.qm_start;
    const int hi = src ? t.qb_end : t.qm_end;
    const u16 *Q = static_cast<const u16 *>(src ? a.qb : a.q);
    const u16 *DO = static_cast<const u16 *>(src ? a.doutb : a.dout);
    const float *LSE = src ? a.lseb : a.lse;
    const int32_t *BOUND = src ? a.bound_branch : a.bound_main;
    const float *DEL = a.delta + (src ? int64_t(a.n_local) * a.hq : 0);
    for (int r0 = lo; r0 < hi; r0 += RB) {
      const int nr = min(RB, hi - r0);
      __syncthreads();  // previous block's LDS reads are done
      // natural Q / dO tiles
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        const int mq = id >> 4, dc = id & 15;
        const int rl = mq >> log2G;
        u32x4 xq = {0, 0, 0, 0}, xd = {0, 0, 0, 0};
        if (rl < nr) {
          const int64_t off = (int64_t(r0 + rl) * a.hq + t.g * G + (mq & (G - 1))) * 128 + dc * 8;
          xq = *reinterpret_cast<const u32x4 *>(Q + off);
          xd = *reinterpret_cast<const u32x4 *>(DO + off);
        }
        *reinterpret_cast<u32x4 *>(sQ + mq * kNatStride + dc * 8) = xq;
        *reinterpret_cast<u32x4 *>(sD + mq * kNatStride + dc * 8) = xd;
      }
      // transposed Q / dO tiles, query slots in kslot16 order
      {
        const int dgrp = tid & 31, qgrp = tid >> 5;
        const int u = qgrp >> 1, sub = qgrp & 1;
        u32x2 vq[8], vd[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int mq = 16 * u + kslot16(8 * sub + jj);
          const int rl = mq >> log2G;
          vq[jj] = u32x2{0, 0};
          vd[jj] = u32x2{0, 0};
          if (rl < nr) {
            const int64_t off =
                (int64_t(r0 + rl) * a.hq + t.g * G + (mq & (G - 1))) * 128 + 4 * dgrp;
            vq[jj] = *reinterpret_cast<const u32x2 *>(Q + off);
            vd[jj] = *reinterpret_cast<const u32x2 *>(DO + off);
          }
        }
        store_t8x4(vq, sQt + (4 * dgrp) * kTrStride + 16 * u + 8 * sub, kTrStride);
        store_t8x4(vd, sDt + (4 * dgrp) * kTrStride + 16 * u + 8 * sub, kTrStride);
      }
      if (tid < kQB) {
        const int rl = tid >> log2G;
        if (rl < nr) {
          const int64_t qh = int64_t(r0 + rl) * a.hq + t.g * G + (tid & (G - 1));
          sL[tid] = LSE[qh] * kLog2e;
          sDel[tid] = DEL[qh];
          sB[tid] = BOUND[r0 + rl];
        } else {
          sL[tid] = 0.f;
          sDel[tid] = 0.f;
          sB[tid] = -1;
        }
      }
      __syncthreads();
      if (!wave_active) continue;

      // a block needs no mask when every row sees every key of the tile
      const bool need_mask =
          !(nr == RB && t.nkeys == kKTileKeys && BOUND[r0] >= t.kpos0 + kKTileKeys - 1);

      // S = Q K^T and dP = dO V^T: 64 queries x this wave's 32 keys
      f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int o0 = qi * kNatStride + ks * 16 + hf * 8;
        const int o1 = (32 + qi) * kNatStride + ks * 16 + hf * 8;
        s0 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sQ + o0)), kreg[ks], s0);
        s1 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sQ + o1)), kreg[ks], s1);
        p0 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sD + o0)), vreg[ks], p0);
        p1 = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sD + o1)), vreg[ks], p1);
      }
      float pr[32], ds[32];
#pragma unroll
      for (int g4 = 0; g4 < 8; ++g4) {
        // queries 32*(g4/4) + 8*(g4%4) + 4*hf + 0..3 are four consecutive slots
        const int q0 = 32 * (g4 >> 2) + 8 * (g4 & 3) + 4 * hf;
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sL + q0);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sDel + q0);
        const int4 b4 = *reinterpret_cast<const int4 *>(sB + q0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g4 + e;
          const float sv = v < 16 ? s0[v] : s1[v - 16];
          const float dpv = v < 16 ? p0[v] : p1[v - 16];
          float p = fast_exp2(sv * sl2 - l4[e]);
          if (need_mask) {
            const int bq = e == 0 ? b4.x : e == 1 ? b4.y : e == 2 ? b4.z : b4.w;
            p = (kvalid && kpos <= bq) ? p : 0.f;
          }
          pr[v] = p;
          ds[v] = p * (dpv - d4[e]);
        }
      }
      bf16x8 pb[4], db[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x4 wp, wd;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          wp[p] = pack_bf2(pr[8 * u + 2 * p], pr[8 * u + 2 * p + 1]);
          wd[p] = pack_bf2(ds[8 * u + 2 * p], ds[8 * u + 2 * p + 1]);
        }
        pb[u] = as_bf16x8(wp);
        db[u] = as_bf16x8(wd);
      }
      // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int o = (32 * dt + qi) * kTrStride + 16 * u + 8 * hf;
          adv[dt] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sDt + o)), pb[u], adv[dt]);
          adk[dt] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sQt + o)), db[u], adk[dt]);
        }
    }
  }

  if (!kvalid) return;
  u16 *DK = static_cast<u16 *>(a.dk);
  u16 *DV = static_cast<u16 *>(a.dv);
  const float sc = a.scale;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d0 = 32 * dt + 8 * a4 + 4 * hf;
      u32x2 wk, wv;
      wk.x = pack_bf2(adk[dt][4 * a4 + 0] * sc, adk[dt][4 * a4 + 1] * sc);
      wk.y = pack_bf2(adk[dt][4 * a4 + 2] * sc, adk[dt][4 * a4 + 3] * sc);
      wv.x = pack_bf2(adv[dt][4 * a4 + 0], adv[dt][4 * a4 + 1]);
      wv.y = pack_bf2(adv[dt][4 * a4 + 2], adv[dt][4 * a4 + 3]);
      *reinterpret_cast<u32x2 *>(DK + koff + d0) = wk;
      *reinterpret_cast<u32x2 *>(DV + koff + d0) = wv;
    }
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const BwdDqArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dq_bf16_kernel, dim3(n_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdDkdvArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dkdv_bf16_kernel, dim3(n_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
