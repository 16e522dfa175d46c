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
//
// Both kernels keep their streamed tiles (K/V, resp. Q/dO) double-buffered
// in LDS in row-major form, load the next tile into registers while the
// current one is computed, and read the operands that are contracted over
// rows (K^T for dQ; Q^T and dO^T for dK/dV) with the LDS transpose read.

#include "kernels.h"
#include "ring_common.h"

namespace ba {

namespace {

constexpr int kBN = 64;  // keys per block in the dQ kernel

// ---------------------------------------------------------------------------
// dQ: query-stationary ring replay

__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(BwdDqArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sK[2][kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV[2][kBN * kRS];

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
  const float c = a.scale_log2;

  int sg, j0;
  Seg s;
  first_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
  const int nseg = 2 * a.C;
  u32x4 RK[4], RV[4];
  if (sg < nseg) {
    load_rows64(RK, K, s, j0, t.g, a.hkv, tid);
    load_rows64(RV, V, s, j0, t.g, a.hkv, tid);
    store_rows64(RK, sK[0], tid);
    store_rows64(RV, sV[0], tid);
  }
  __syncthreads();
  int cur = 0;
  while (sg < nseg) {
    const Seg cs = s;
    const int cj0 = j0;
    next_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
    const bool more = sg < nseg;
    if (more) {
      load_rows64(RK, K, s, j0, t.g, a.hkv, tid);
      load_rows64(RV, V, s, j0, t.g, a.hkv, tid);
    }
    if (wave_active) {
      const u16 *bk = sK[cur];
      const u16 *bv = sV[cur];
      // S^T = K Q^T and dP^T = V dO^T for 64 keys
      f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s0 = mfma32(lds_nat(bk, 0, ks * 16, lane), qreg[ks], s0);
        s1 = mfma32(lds_nat(bk, 32, ks * 16, lane), qreg[ks], s1);
        p0 = mfma32(lds_nat(bv, 0, ks * 16, lane), dreg[ks], p0);
        p1 = mfma32(lds_nat(bv, 32, ks * 16, lane), dreg[ks], p1);
      }
      const bool need_mask = cj0 + kBN > cs.n_full;
      float ds[32];
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const float sv = v < 16 ? s0[v] : s1[v - 16];
        const float dpv = v < 16 ? p0[v] : p1[v - 16];
        float p = fast_exp2(fmaf(sv, c, -lse2));
        if (need_mask) {
          const int jj = cj0 + 32 * (v >> 4) + 8 * ((v & 15) >> 2) + 4 * hf + (v & 3);
          const bool vis = (jj < cs.n_hi) && (cs.cpos0 + jj <= bound);
          p = vis ? p : 0.f;
        }
        ds[v] = p * (dpv - delta);
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 db = pack8(ds + 8 * u);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma32(lds_tr(bk, 16 * u, 32 * dt, lane), db, acc[dt]);
      }
    }
    if (more) {
      store_rows64(RK, sK[cur ^ 1], tid);
      store_rows64(RV, sV[cur ^ 1], tid);
    }
    __syncthreads();
    cur ^= 1;
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
      w.x = cvt_pk_bf16(x0, x1);
      w.y = cvt_pk_bf16(x2, x3);
      *reinterpret_cast<u32x2 *>(DQ + qh * 128 + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// dK / dV: key-stationary ring replay

constexpr int kQB = 64;  // query vectors per inner block

struct QBlockRegs {
  u32x4 q[4], d[4];
  float l, del;
  int b;
};

// Inner blocks are numbered over the main-row range then the branch-row range.
struct QBlock {
  int src, r0, nr;
};

__device__ __forceinline__ QBlock qblock(const KTile &t, int b, int RB, int nb_main) {
  QBlock q;
  if (b < nb_main) {
    q.src = 0;
    q.r0 = t.qm_start + b * RB;
    q.nr = min(RB, t.qm_end - q.r0);
  } else {
    q.src = 1;
    q.r0 = t.qb_start + (b - nb_main) * RB;
    q.nr = min(RB, t.qb_end - q.r0);
  }
  return q;
}

__device__ __forceinline__ void qblock_load(QBlockRegs &R, const BwdDkdvArgs &a, const KTile &t,
                                            const QBlock &qb, int tid) {
  const u16 *Q = static_cast<const u16 *>(qb.src ? a.qb : a.q);
  const u16 *DO = static_cast<const u16 *>(qb.src ? a.doutb : a.dout);
  const int G = a.G, log2G = a.log2G;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int mq = id >> 4, dc = id & 15;
    const int rl = mq >> log2G;
    R.q[i] = u32x4{0, 0, 0, 0};
    R.d[i] = u32x4{0, 0, 0, 0};
    if (rl < qb.nr) {
      const int64_t off = (int64_t(qb.r0 + rl) * a.hq + t.g * G + (mq & (G - 1))) * 128 + dc * 8;
      R.q[i] = *reinterpret_cast<const u32x4 *>(Q + off);
      R.d[i] = *reinterpret_cast<const u32x4 *>(DO + off);
    }
  }
  if (tid < kQB) {
    const int rl = tid >> log2G;
    R.l = 0.f;
    R.del = 0.f;
    R.b = -1;
    if (rl < qb.nr) {
      const int64_t qh = int64_t(qb.r0 + rl) * a.hq + t.g * G + (tid & (G - 1));
      R.l = (qb.src ? a.lseb : a.lse)[qh] * kLog2e;
      R.del = a.delta[(qb.src ? int64_t(a.n_local) * a.hq : 0) + qh];
      R.b = (qb.src ? a.bound_branch : a.bound_main)[qb.r0 + rl];
    }
  }
}

__device__ __forceinline__ void qblock_store(const QBlockRegs &R, u16 *sQ, u16 *sD, float *sL,
                                             float *sDel, int *sB, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int mq = id >> 4, dc = id & 15;
    *reinterpret_cast<u32x4 *>(sQ + mq * kRS + dc * 8) = R.q[i];
    *reinterpret_cast<u32x4 *>(sD + mq * kRS + dc * 8) = R.d[i];
  }
  if (tid < kQB) {
    sL[tid] = R.l;
    sDel[tid] = R.del;
    sB[tid] = R.b;
  }
}

__global__ __launch_bounds__(256) void bwd_dkdv_bf16_kernel(BwdDkdvArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sQ[2][kQB * kRS];
  __shared__ __attribute__((aligned(16))) u16 sD[2][kQB * kRS];
  __shared__ __attribute__((aligned(16))) float sL[2][kQB];
  __shared__ __attribute__((aligned(16))) float sDel[2][kQB];
  __shared__ __attribute__((aligned(16))) int sB[2][kQB];

  const KTile t = a.ktiles[blockIdx.x];
  if (t.nkeys == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hf = lane >> 5;
  const int kk = wave * 32 + qi;  // this lane's key inside the tile
  const bool kvalid = kk < t.nkeys;
  const int kpos = t.kpos0 + kk;
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
  const float c = a.scale_log2;
  const int RB = kQB >> a.log2G;  // rows per inner block
  const bool wave_active = (wave * 32) < t.nkeys;
  const int nb_main = (t.qm_end - t.qm_start + RB - 1) / RB;
  const int nb = nb_main + (t.qb_end - t.qb_start + RB - 1) / RB;

  QBlockRegs R;
  if (nb > 0) {
    qblock_load(R, a, t, qblock(t, 0, RB, nb_main), tid);
    qblock_store(R, sQ[0], sD[0], sL[0], sDel[0], sB[0], tid);
  }
  __syncthreads();
  int cur = 0;
  for (int b = 0; b < nb; ++b) {
    const QBlock qb = qblock(t, b, RB, nb_main);
    const bool more = b + 1 < nb;
    if (more) qblock_load(R, a, t, qblock(t, b + 1, RB, nb_main), tid);
    if (wave_active) {
      const u16 *bq = sQ[cur];
      const u16 *bd = sD[cur];
      const int32_t *BOUND = qb.src ? a.bound_branch : a.bound_main;
      // no mask when every row of the block sees every key of the tile
      const bool need_mask =
          !(qb.nr == RB && t.nkeys == kKTileKeys && BOUND[qb.r0] >= t.kpos0 + kKTileKeys - 1);
      // S = Q K^T and dP = dO V^T: 64 queries x this wave's 32 keys
      f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s0 = mfma32(lds_nat(bq, 0, ks * 16, lane), kreg[ks], s0);
        s1 = mfma32(lds_nat(bq, 32, ks * 16, lane), kreg[ks], s1);
        p0 = mfma32(lds_nat(bd, 0, ks * 16, lane), vreg[ks], p0);
        p1 = mfma32(lds_nat(bd, 32, ks * 16, lane), vreg[ks], p1);
      }
      float pr[32], ds[32];
#pragma unroll
      for (int g4 = 0; g4 < 8; ++g4) {
        // queries 32*(g4/4) + 8*(g4%4) + 4*hf + 0..3 are four consecutive slots
        const int q0 = 32 * (g4 >> 2) + 8 * (g4 & 3) + 4 * hf;
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sL[cur] + q0);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sDel[cur] + q0);
        const int4 b4 = *reinterpret_cast<const int4 *>(sB[cur] + q0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g4 + e;
          const float sv = v < 16 ? s0[v] : s1[v - 16];
          const float dpv = v < 16 ? p0[v] : p1[v - 16];
          float p = fast_exp2(fmaf(sv, c, -l4[e]));
          if (need_mask) {
            const int bq4 = e == 0 ? b4.x : e == 1 ? b4.y : e == 2 ? b4.z : b4.w;
            p = (kvalid && kpos <= bq4) ? p : 0.f;
          }
          pr[v] = p;
          ds[v] = p * (dpv - d4[e]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 pb = pack8(pr + 8 * u);
        const bf16x8 db = pack8(ds + 8 * u);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          adv[dt] = mfma32(lds_tr(bd, 16 * u, 32 * dt, lane), pb, adv[dt]);
          adk[dt] = mfma32(lds_tr(bq, 16 * u, 32 * dt, lane), db, adk[dt]);
        }
      }
    }
    if (more) qblock_store(R, sQ[cur ^ 1], sD[cur ^ 1], sL[cur ^ 1], sDel[cur ^ 1], sB[cur ^ 1], tid);
    __syncthreads();
    cur ^= 1;
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
      wk.x = cvt_pk_bf16(adk[dt][4 * a4 + 0] * sc, adk[dt][4 * a4 + 1] * sc);
      wk.y = cvt_pk_bf16(adk[dt][4 * a4 + 2] * sc, adk[dt][4 * a4 + 3] * sc);
      wv.x = cvt_pk_bf16(adv[dt][4 * a4 + 0], adv[dt][4 * a4 + 1]);
      wv.y = cvt_pk_bf16(adv[dt][4 * a4 + 2], adv[dt][4 * a4 + 3]);
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
