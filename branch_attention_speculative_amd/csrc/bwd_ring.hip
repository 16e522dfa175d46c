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
// in LDS in row-major form, load the next tile straight from global memory
// into the idle buffer while the current one is computed, and read the
// operands that are contracted over rows (K^T for dQ; Q^T and dO^T for
// dK/dV) with the LDS transpose read. P is recomputed from LSE * log2(e),
// which the backward preprocess stores next to Delta.

#include "kernels.h"
#include "ring_common.h"

namespace ba {

namespace {

constexpr int kBN = 64;  // keys per block in the dQ kernel

// ---------------------------------------------------------------------------
// dQ: query-stationary ring replay

// One 64-key block, one 32-key tile at a time: S^T = K Q^T, dP^T = V dO^T,
// dS = P (dP - Delta), dQ^T += K^T dS^T. When the block crosses a causal
// bound or the chunk's visible end (need_mask), scores of keys past lim (the
// last visible key for this lane, relative to the block, minus 4 hf) are
// set to -inf before the exponentials.
template <bool QK8>
__device__ __forceinline__ void dq_block(f32x16 (&acc)[4], const bf16x8 (&qreg)[8],
                                         const i32x8 (&q8)[2], const bf16x8 (&dreg)[8],
                                         const u16 *bk, const u16 *bk8, const u16 *bv,
                                         bool need_mask, int lim, float lse2, const f32x16 &ndelta,
                                         float c, const NatOff &no, const Nat8Off &no8,
                                         const TrOff &to) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    // dP^T accumulates onto -Delta, so it comes out as dP - Delta
    f32x16 s = f32x16{}, p = ndelta;
    if constexpr (QK8) {  // S^T from the E4M3 K tile and Q registers
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) s = mfma32_f8(lds_nat8(bk8, 32 * kt, kk, no8), q8[kk], s);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (!QK8) s = mfma32(lds_nat_o(bk, 32 * kt, ks, no), qreg[ks], s);
      p = mfma32(lds_nat_o(bv, 32 * kt, ks, no), dreg[ks], p);
    }
    if (need_mask) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int jj = 32 * kt + 8 * (v >> 2) + (v & 3);
        s[v] = jj <= lim ? s[v] : kNegInf;
      }
    }
    float ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) ds[v] = fast_exp2(fmaf(s[v], c, -lse2)) * p[v];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const bf16x8 db = pack8(ds + 8 * w);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma32(lds_tr_o(bk, 32 * kt + 16 * w, dt, to), db, acc[dt]);
    }
  }
}

constexpr int kDqWaves = 8;  // waves per dQ workgroup (32 query vectors each)

// RUNS: walk the tile's run list (else the segments). QK8: the scores come
// from the fp8 matrix cores on the E4M3 Q and K (an fp8 plan), which halves
// their share of the matrix-core time; K^T dS^T still takes the exact bf16
// copy of K.
template <bool RUNS, bool QK8>
__global__ __launch_bounds__(kDqWaves * 64, 1) void bwd_dq_bf16_kernel(BwdDqArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sK0[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV0[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sK1[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV1[kBN * kRS];
  // E4M3 K tiles: 64 rows of 128 bytes
  __shared__ __attribute__((aligned(16))) u16 sK80[QK8 ? kBN * 64 : 8];
  __shared__ __attribute__((aligned(16))) u16 sK81[QK8 ? kBN * 64 : 8];
  __shared__ __attribute__((aligned(16))) RunSeg sRuns[RUNS ? kMaxRuns : 1];
  __shared__ int sNRuns;

  const QTile t = a.qtiles[blockIdx.x];
  if (t.nrows == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform_int(tid >> 6);
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
  const int64_t qall = (t.src ? int64_t(a.n_local) * a.hq : 0) + qh;
  const float lse2 = (bound >= 0) ? a.lse2[qall] : 0.f;
  const float ndel = (bound >= 0) ? a.ndelta[qall] : 0.f;

  bf16x8 qreg[8], dreg[8];
  i32x8 q8[2];
  {
    const u16 *qp = Q + qh * 128 + hf * 8;
    const u16 *dp = DO + qh * 128 + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (!QK8)
        qreg[ks] = as_bf16x8(valid ? *reinterpret_cast<const u32x4 *>(qp + ks * 16) : u32x4{0, 0, 0, 0});
      dreg[ks] = as_bf16x8(valid ? *reinterpret_cast<const u32x4 *>(dp + ks * 16) : u32x4{0, 0, 0, 0});
    }
    if constexpr (QK8) {
      // E4M3 rows are 128 bytes: this lane's bytes 64 kk + 32 hf .. + 31
      const char *q8p = static_cast<const char *>(t.src ? a.qb8 : a.q8) + qh * 128 + hf * 32;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 lo = valid ? *reinterpret_cast<const u32x4 *>(q8p + 64 * kk) : u32x4{0, 0, 0, 0};
        const u32x4 hi = valid ? *reinterpret_cast<const u32x4 *>(q8p + 64 * kk + 16) : u32x4{0, 0, 0, 0};
        q8[kk] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                       int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      }
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  const float c = a.scale_log2;
  const int64_t rs = int64_t(a.hkv) * 128;
  const int g = t.g;

  const NatOff no = nat_offsets(lane);
  const Nat8Off no8 = nat8_offsets(lane);
  const TrOff to = tr_offsets(lane);
  const DmaOff<kDqWaves> dof =
      dma_offsets<kDqWaves>(wave, lane, [&](int r) { return int64_t(r) * rs; });
  // E4M3 K: rows of hkv * 128 bytes
  const uint32_t dof8 = dma8_offset(wave, lane, rs);
  const char *K8 = static_cast<const char *>(a.k8);
  // K/V rows j0 .. j0 + 63 of a chunk; rows past the chunk's visible end
  // are not read (their P is masked to zero)
  auto dma_kv = [&](const Seg &s, int j0, u16 *dk, u16 *dv, u16 *dk8) {
    const int64_t off = (s.krow + j0) * rs + g * 128;
    const uint32_t bytes = uint32_t(((min(kBN, s.n_hi - j0) - 1) * rs + 128) * 2);
    dma_tile64_buf<kDqWaves>(dk, buf_rsrc(K + off, bytes), dof, wave);
    dma_tile64_buf<kDqWaves>(dv, buf_rsrc(V + off, bytes), dof, wave);
    // same rows at one byte per element: the element offset is the byte
    // offset, and the extent is half the bf16 one
    if constexpr (QK8) dma_tile64_f8(dk8, buf_rsrc(K8 + off, bytes / 2), dof8, wave);
  };
  f32x16 ndelta;
#pragma unroll
  for (int v = 0; v < 16; ++v) ndelta[v] = ndel;

  lds_zero(sK0, kBN * kRS, tid, kDqWaves * 64);
  lds_zero(sV0, kBN * kRS, tid, kDqWaves * 64);
  lds_zero(sK1, kBN * kRS, tid, kDqWaves * 64);
  lds_zero(sV1, kBN * kRS, tid, kDqWaves * 64);
  if constexpr (QK8) {
    lds_zero(sK80, kBN * 64, tid, kDqWaves * 64);
    lds_zero(sK81, kBN * 64, tid, kDqWaves * 64);
  }
  if constexpr (RUNS) {
    if (wave == 0) build_runs(sRuns, &sNRuns, t, a.C, a.r, a.n_local, lane);
  }
  __syncthreads();

  int sg, j0;
  Seg s;
  int nseg = 2 * a.C;  // end of the walk: segments, or runs
  if constexpr (RUNS) {
    nseg = uniform_int(sNRuns);
    first_run(sg, j0, s, sRuns, nseg);
  } else {
    first_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
  }
  auto advance = [&]() {
    if constexpr (RUNS)
      next_run<kBN>(sg, j0, s, sRuns, nseg);
    else
      next_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
  };
  if (sg < nseg) dma_kv(s, j0, sK0, sV0, sK80);
  dma_wait();
  __syncthreads();
  while (sg < nseg) {
    {
      const Seg cs = s;
      const int cj0 = j0;
      advance();
      if (sg < nseg) dma_kv(s, j0, sK1, sV1, sK81);
      if (wave_active) {
        const bool need = cj0 + kBN > cs.n_full;
        const int lim = min(cs.n_hi - 1, bound - cs.cpos0) - cj0 - 4 * hf;
        dq_block<QK8>(acc, qreg, q8, dreg, sK0, sK80, sV0, need, lim, lse2, ndelta, c, no, no8, to);
      }
      dma_wait();
      __syncthreads();
    }
    if (sg >= nseg) break;
    {
      const Seg cs = s;
      const int cj0 = j0;
      advance();
      if (sg < nseg) dma_kv(s, j0, sK0, sV0, sK80);
      if (wave_active) {
        const bool need = cj0 + kBN > cs.n_full;
        const int lim = min(cs.n_hi - 1, bound - cs.cpos0) - cj0 - 4 * hf;
        dq_block<QK8>(acc, qreg, q8, dreg, sK1, sK81, sV1, need, lim, lse2, ndelta, c, no, no8, to);
      }
      dma_wait();
      __syncthreads();
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
      w.x = cvt_pk_bf16(x0, x1);
      w.y = cvt_pk_bf16(x2, x3);
      *reinterpret_cast<u32x2 *>(DQ + qh * 128 + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// dK / dV: key-stationary ring replay

constexpr int kQB = 64;  // query vectors per inner block

// Inner blocks are numbered over the branch-row range, then the main-row
// range, each walked from its end backwards in blocks that end on a multiple
// of RB rows from the range end (the partial block, which holds the range's
// first rows, comes last). Every key tile of a kv-head ends its ranges on
// the same rows, so the tiles that start together on an XCD read the same
// Q / dO rows at about the same time and share them in L2: on the long
// workload this halves the kernel's HBM reads against walking forward from
// each tile's own first row.
struct QBlock {
  int src, r0, nr, hi;
};

__device__ __forceinline__ QBlock qblock(const KTile &t, int b, int RB, int nb_main) {
  const int nb_branch = (t.qb_end - t.qb_start + RB - 1) / RB;
  QBlock q;
  int lo, end, k;
  if (b < nb_branch) {
    q.src = 1;
    lo = t.qb_start;
    end = t.qb_end;
    k = b;
  } else {
    q.src = 0;
    lo = t.qm_start;
    end = t.qm_end;
    k = b - nb_branch;
  }
  q.hi = end - k * RB;  // one past the block's last row
  q.r0 = max(q.hi - RB, lo);
  q.nr = q.hi - q.r0;
  return q;
}

// The eight waves of a dK/dV workgroup come in pairs that own the same 32
// keys and sit on the same SIMD. The first wave of a pair computes S = Q K^T,
// P = exp(S - LSE) and dV^T += dO^T P; it also hands P (bf16, in its MFMA
// register layout) to its partner through LDS. The partner runs one inner
// block behind: it computes dP = dO V^T and dS = P (dP - Delta) with the P
// its partner published in the previous block, and dK^T += Q^T dS. Each wave
// then needs about half the registers of one wave doing all four products,
// so two waves fit on each SIMD, with no duplicated products and a single
// barrier per block.

constexpr int kXchg = 4 * 64 * 4;  // u32 per wave pair: 4 bf16x8 operands x 64 lanes

// dV wave, phase 1 of a block: S and P for 64 query vectors; P goes to the
// exchange slot (xs) and stays in pb for phase 2.
template <bool MASK>
__device__ __forceinline__ void dv_phase1(bf16x8 (&pb)[4], const bf16x8 (&kreg)[8], const u16 *bq,
                                          const float *sl, const int *sb, uint32_t *xs, int nvalid,
                                          bool kvalid, int kpos, float c, int lane, int hf,
                                          const NatOff &no) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s = mfma32(lds_nat_o(bq, 32 * mt, ks, no), kreg[ks], s);
    float pr[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // queries 32 mt + 8 g4 + 4 hf + 0..3 are four consecutive slots
      const int q0 = 32 * mt + 8 * g4 + 4 * hf;
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sl + q0);
      int4 b4 = {0, 0, 0, 0};
      if (MASK) b4 = *reinterpret_cast<const int4 *>(sb + q0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = fast_exp2(fmaf(s[4 * g4 + e], c, -l4[e]));
        if (MASK) {
          const int bq4 = e == 0 ? b4.x : e == 1 ? b4.y : e == 2 ? b4.z : b4.w;
          pv = (kvalid && q0 + e < nvalid && kpos <= bq4) ? pv : 0.f;
        }
        pr[4 * g4 + e] = pv;
      }
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int u = 2 * mt + w;
      pb[u] = pack8(pr + 8 * w);
      *reinterpret_cast<u32x4 *>(xs + (u * 64 + lane) * 4) = __builtin_bit_cast(u32x4, pb[u]);
    }
  }
}

// dV wave, phase 2: dV^T += dO^T P.
__device__ __forceinline__ void dv_phase2(f32x16 (&adv)[4], const bf16x8 (&pb)[4], const u16 *bd,
                                          const TrOff &to) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) adv[dt] = mfma32(lds_tr_o(bd, 16 * u, dt, to), pb[u], adv[dt]);
}

// dK wave, phase 1: dP - Delta = dO V^T - Delta for 64 query vectors (the
// product accumulates onto -Delta of each row, from LDS snd).
__device__ __forceinline__ void dk_phase1(f32x16 (&dp)[2], const bf16x8 (&vreg)[8], const u16 *bd,
                                          const float *snd, int hf, const NatOff &no) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x16 p;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // rows 32 mt + 8 g4 + 4 hf + 0..3 are four consecutive slots
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(snd + 32 * mt + 8 * g4 + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[4 * g4 + e] = d4[e];
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) p = mfma32(lds_nat_o(bd, 32 * mt, ks, no), vreg[ks], p);
    dp[mt] = p;
  }
}

// dK wave, phase 2: dS = P (dP - Delta) with P from the exchange slot,
// dK^T += Q^T dS.
__device__ __forceinline__ void dk_phase2(f32x16 (&adk)[4], const f32x16 (&dp)[2], const u16 *bq,
                                          const uint32_t *xs, int lane, const TrOff &to) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    float ds[16];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const u32x4 pw = *reinterpret_cast<const u32x4 *>(xs + ((2 * mt + w) * 64 + lane) * 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ds[8 * w + 2 * k] = __uint_as_float(pw[k] << 16);
        ds[8 * w + 2 * k + 1] = __uint_as_float(pw[k] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) ds[v] *= dp[mt][v];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const bf16x8 db = pack8(ds + 8 * w);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        adk[dt] = mfma32(lds_tr_o(bq, 16 * (2 * mt + w), dt, to), db, adk[dt]);
    }
  }
}

__global__ __launch_bounds__(512) void bwd_dkdv_bf16_kernel(BwdDkdvArgs a) {
  // Q / dO tiles and the per-row LSE, Delta and bounds of an inner block,
  // three sets: the dV waves work on block b while the dK waves work on
  // block b - 1 and block b + 1 is loading. Separate objects so the LDS loads
  // into one set never order the reads of another.
  __shared__ __attribute__((aligned(16))) u16 sQ0[kQB * kRS];
  __shared__ __attribute__((aligned(16))) u16 sD0[kQB * kRS];
  __shared__ __attribute__((aligned(16))) u16 sQ1[kQB * kRS];
  __shared__ __attribute__((aligned(16))) u16 sD1[kQB * kRS];
  __shared__ __attribute__((aligned(16))) u16 sQ2[kQB * kRS];
  __shared__ __attribute__((aligned(16))) u16 sD2[kQB * kRS];
  __shared__ __attribute__((aligned(16))) float sL0[kQB], sE0[kQB], sL1[kQB], sE1[kQB], sL2[kQB],
      sE2[kQB];
  __shared__ __attribute__((aligned(16))) int sB0[kQB], sB1[kQB], sB2[kQB];
  // P exchange of each wave pair, one slot per set (block b uses slot b % 3)
  __shared__ __attribute__((aligned(16))) uint32_t sX0[4 * kXchg];
  __shared__ __attribute__((aligned(16))) uint32_t sX1[4 * kXchg];
  __shared__ __attribute__((aligned(16))) uint32_t sX2[4 * kXchg];

  const KTile t = a.ktiles[blockIdx.x];
  if (t.nkeys == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform_int(tid >> 6);
  const int role = wave >> 2;  // 0: S, P, dV wave; 1: dP, dS, dK wave
  const int qi = lane & 31, hf = lane >> 5;
  const int kk = (wave & 3) * 32 + qi;  // this lane's key inside the tile
  const bool kvalid = kk < t.nkeys;
  const int kpos = t.kpos0 + kk;
  int64_t krow;
  if (t.run > 0) {  // packed joined runs of consecutive shards
    const int v = t.run_off + min(kk, t.nkeys - 1);
    krow = int64_t(t.shard + v / t.run) * a.n_local + t.krow0 + v % t.run;
  } else {
    krow = int64_t(t.shard) * a.n_local + t.krow0 + min(kk, t.nkeys - 1);
  }
  const int64_t koff = (krow * a.hkv + t.g) * 128;
  const int G = a.G, log2G = a.log2G;
  const float c = a.scale_log2;
  const int RB = kQB >> log2G;  // rows per inner block
  const bool wave_active = ((wave & 3) * 32) < t.nkeys;
  const int nb_main = (t.qm_end - t.qm_start + RB - 1) / RB;
  const int nb = nb_main + (t.qb_end - t.qb_start + RB - 1) / RB;
  const int hq = a.hq;
  const int xo = (wave & 3) * kXchg;  // this pair's part of an exchange slot

  const NatOff no = nat_offsets(lane);
  const TrOff to = tr_offsets(lane);
  // tile row mq is query vector (row r0 + mq / G, head g G + mq % G)
  const DmaOff<4> dof = dma_offsets<4>(
      wave & 3, lane, [&](int mq) { return (int64_t(mq >> log2G) * hq + (mq & (G - 1))) * 128; });
  // Issue the loads of inner block b into one buffer set. Only the four dV
  // waves (0-3) load: the per-row data first (waves 1-3), then the Q / dO
  // tiles (all four). The dK waves, one block behind, issue no loads; this
  // measured about 4% faster than all eight waves sharing the tile loads.
  auto dma_block = [&](int b, u16 *dq, u16 *dd, float *dl, float *de, int *db) {
    const QBlock qb = qblock(t, b, RB, nb_main);
    const int hb = t.g * G;
    const int64_t base = qb.src ? int64_t(a.n_local) * hq : 0;
    const int rr = min(qb.r0 + (lane >> log2G), qb.hi - 1);
    const int64_t qh = base + int64_t(rr) * hq + hb + (lane & (G - 1));
    if (wave == 1) dma_dword64(dl, a.lse2 + qh);
    if (wave == 2) dma_dword64(de, a.ndelta + qh);
    if (wave == 3) dma_dword64(db, (qb.src ? a.bound_branch : a.bound_main) + rr);
    if (wave < 4) {
      const u16 *Q = static_cast<const u16 *>(qb.src ? a.qb : a.q);
      const u16 *DO = static_cast<const u16 *>(qb.src ? a.doutb : a.dout);
      // query vectors past the range are not read (their P is masked to zero)
      const int64_t off = (int64_t(qb.r0) * hq + hb) * 128;
      const uint32_t bytes = uint32_t(((int64_t(qb.nr - 1) * hq + G - 1) * 128 + 128) * 2);
      dma_tile64_buf<4>(dq, buf_rsrc(Q + off, bytes), dof, wave);
      dma_tile64_buf<4>(dd, buf_rsrc(DO + off, bytes), dof, wave);
    }
  };
  // no mask when every row of the block sees every key of the tile; rows
  // are in increasing bound order, so the first row's bound (sb[0], the
  // block's bounds in LDS) decides
  auto need_mask = [&](int b, const int *sb) {
    const QBlock qb = qblock(t, b, RB, nb_main);
    return !(qb.nr == RB && t.nkeys == kKTileKeys && sb[0] >= t.kpos0 + kKTileKeys - 1);
  };
  auto nvalid = [&](int b) { return qblock(t, b, RB, nb_main).nr << log2G; };

  // operand registers: K for the S wave, V for the dP wave
  const u16 *KV = static_cast<const u16 *>(role ? a.v : a.k);
  bf16x8 kvreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    kvreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(KV + koff + ks * 16 + hf * 8));
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  lds_zero(sQ0, kQB * kRS, tid, 512);
  lds_zero(sD0, kQB * kRS, tid, 512);
  lds_zero(sQ1, kQB * kRS, tid, 512);
  lds_zero(sD1, kQB * kRS, tid, 512);
  lds_zero(sQ2, kQB * kRS, tid, 512);
  lds_zero(sD2, kQB * kRS, tid, 512);
  __syncthreads();

  // Iteration b = 0 .. nb: one barrier, then the dV waves issue the loads of
  // block b + 1 and do block b (S, P -> exchange slot b % 3, dV) while the
  // dK waves do block b - 1 (dP, dS with P from slot (b - 1) % 3, dK). The barrier at
  // the top of iteration b publishes block b's tiles and P of block b - 1,
  // and frees the set and slot that iteration b + 1 overwrites.
  if (nb > 0) dma_block(0, sQ0, sD0, sL0, sE0, sB0);
  dma_wait();
  // The two roles run separate loops with the same barrier sequence.
  if (role == 0) {
    // The dV wave is the one its partner waits for at the barrier: it issues
    // first when both have an instruction ready (0.26% faster on long256k;
    // the opposite priority is 5% slower).
    __builtin_amdgcn_s_setprio(1);
    // block b in the set (Qc, Dc, Lc, Bc); block b + 1 loads into the next set
    auto iter = [&](int b, const u16 *Qc, const u16 *Dc, const float *Lc, const int *Bc, uint32_t *Xc,
                    u16 *Qn, u16 *Dn, float *Ln, float *En, int *Bn) {
      __syncthreads();
      const bool mask = b < nb && need_mask(b, Bc);
      if (b + 1 < nb) dma_block(b + 1, Qn, Dn, Ln, En, Bn);
      if (wave_active && b < nb) {
        uint32_t *xs = Xc + xo;
        bf16x8 pb[4];
        if (mask)
          dv_phase1<true>(pb, kvreg, Qc, Lc, Bc, xs, nvalid(b), kvalid, kpos, c, lane, hf, no);
        else
          dv_phase1<false>(pb, kvreg, Qc, Lc, Bc, xs, nvalid(b), kvalid, kpos, c, lane, hf, no);
        dv_phase2(acc, pb, Dc, to);
      }
      dma_wait();
    };
    for (int b = 0; b <= nb; b += 3) {
      iter(b, sQ0, sD0, sL0, sB0, sX0, sQ1, sD1, sL1, sE1, sB1);
      if (b + 1 > nb) break;
      iter(b + 1, sQ1, sD1, sL1, sB1, sX1, sQ2, sD2, sL2, sE2, sB2);
      if (b + 2 > nb) break;
      iter(b + 2, sQ2, sD2, sL2, sB2, sX2, sQ0, sD0, sL0, sE0, sB0);
    }
  } else {
    // block b - 1 in the set (Qp, Dp, Ep)
    auto iter = [&](int b, const u16 *Qp, const u16 *Dp, const float *Ep, const uint32_t *Xp) {
      __syncthreads();
      if (wave_active && b >= 1) {
        const uint32_t *xs = Xp + xo;  // P of block b - 1
        f32x16 dp[2];
        dk_phase1(dp, kvreg, Dp, Ep, hf, no);
        dk_phase2(acc, dp, Qp, xs, lane, to);
      }
    };
    for (int b = 0; b <= nb; b += 3) {
      iter(b, sQ2, sD2, sE2, sX2);
      if (b + 1 > nb) break;
      iter(b + 1, sQ0, sD0, sE0, sX0);
      if (b + 2 > nb) break;
      iter(b + 2, sQ1, sD1, sE1, sX1);
    }
  }

  if (!kvalid) return;
  u16 *OUT = static_cast<u16 *>(role ? a.dk : a.dv);
  const float sc = role ? a.scale : 1.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d0 = 32 * dt + 8 * a4 + 4 * hf;
      u32x2 w;
      w.x = cvt_pk_bf16(acc[dt][4 * a4 + 0] * sc, acc[dt][4 * a4 + 1] * sc);
      w.y = cvt_pk_bf16(acc[dt][4 * a4 + 2] * sc, acc[dt][4 * a4 + 3] * sc);
      *reinterpret_cast<u32x2 *>(OUT + koff + d0) = w;
    }
}

template __global__ void bwd_dq_bf16_kernel<false, false>(BwdDqArgs);
template __global__ void bwd_dq_bf16_kernel<true, false>(BwdDqArgs);
template __global__ void bwd_dq_bf16_kernel<false, true>(BwdDqArgs);
template __global__ void bwd_dq_bf16_kernel<true, true>(BwdDqArgs);

}  // namespace

hipError_t launch_bwd_dq_bf16(const BwdDqArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  const dim3 g(n_tiles), b(kDqWaves * 64);
  if (a.k8 != nullptr) {
    if (a.runs)
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<true, true>), g, b, 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<false, true>), g, b, 0, s, a);
  } else if (a.runs) {
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<true, false>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<false, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdDkdvArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dkdv_bf16_kernel, dim3(n_tiles), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
