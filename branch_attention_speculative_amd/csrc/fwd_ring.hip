// Ring-step causal partial, forward (bf16 in, fp32 accumulate, D = 128).
//
// One workgroup (8 waves) owns a query tile: up to 256 query vectors
// (consecutive rows of one sequence chunk x the G q-heads of one kv-head). It
// walks the virtual ring i = 0..C-1 over shard (r - i) mod C -- the K/V that
// would circulate while the queries stay (ai.info summary, Methodology;
// rainbus analysis, method steps, step two) -- and inside each shard the
// sequence's head chunk, then its tail chunk, in blocks of 64 keys. The
// online-softmax state (running max, sum, unnormalised O) is carried in
// registers across blocks and ring steps, which is the log-sum-exp merge
// between ring steps (rainbus analysis, core method, Eq. 2, applied
// incrementally). Key blocks past a tile's largest causal bound are never
// visited; blocks wholly inside its smallest bound skip the mask.
//
// Per wave: 32 query vectors. Scores are formed transposed, S^T = K Q^T, so a
// lane owns one query; O^T += V^T P^T takes P^T straight from the score
// registers, and V^T is read from the row-major V tile with the LDS
// transpose read, in the key order the score registers come in.
//
// Vector-unit work is the scarce resource next to the matrix cores (on
// gfx950 at most about a fifth of the matrix-core time on a SIMD can carry
// vector instructions; beyond that every one of them costs matrix-core
// time), so the softmax keeps it to about three and a half
// instructions per score (scale-and-subtract, exp2, add, half a pack): the
// running max is the exact max of the first block only and afterwards moves
// only when a block's exponentials overflow 2^64 (checked once per block on
// their sum; that block is then redone with its exact max). The sum of P
// stays in fp32: summing the bf16-rounded P would cost the LSE up to 2^-9
// relative on rows that see few keys.
//
// K and V tiles are double-buffered in LDS and the next block is loaded
// straight from global memory into the idle buffers while the current one
// is computed (one barrier per block). Eight waves share each tile, which
// halves the tile traffic into LDS per product compared with four.

//
// The fp8 instance (template flag QK8) takes Q and K as OCP fp8 E4M3 codes
// and forms the scores with the gfx950 fp8 matrix-core product
// (32x32x64, fp32 accumulate: two products per 32-key tile over D = 128
// instead of eight bf16 ones); V, P, O and the softmax are the bf16
// instance's. A K tile is then 64 rows of 128 bytes in LDS, swizzled by its
// own rule (fp8 K tile layout below).

#include "kernels.h"
#include "ring_common.h"

namespace ba {

namespace {

constexpr int kBN = 64;  // keys per block
constexpr float kOver = 18446744073709551616.f;  // 2^64: largest sum of P per lane and block


struct FwdState {
  bf16x8 qreg[8];  // bf16 instance: Q^T operands, 8 steps of 16 of D
  i32x8 q8[2];     // fp8 instance: Q^T operands, 2 steps of 64 of D
  f32x16 acc[4];
  float mrun, lsum;
};

// Block of the ring walk: segment sg (with its chunk info) and first key j0
// inside the chunk.
struct Blk {
  int sg, j0;
  Seg s;
};

// What the block loop needs of a block.
struct BlkRec {
  int64_t off;     // element offset of its first key row (kv-head included)
  uint32_t bytes;  // extent of its visible rows in bytes; 0: no such block
  int lim;         // last key of the block any row of the tile sees
  int pos0;        // sequence position of its first key
  int need;        // some row of the tile does not see every key of it
};

// Scores of one 64-key block: two 32-key MFMA tiles; element v of the block
// is x[v / 16][v % 16].
typedef f32x16 Scores[2];

// S^T = K Q^T for one 64-key block. The K operands of step ks + 1 are read
// from LDS before the products of step ks, and the scheduling barrier keeps
// the compiler from sinking them back next to their use (measured about 1%
// faster on the long workload than reading each operand just before its
// product).
__device__ __forceinline__ void scores(Scores &x, const u16 *bk, const FwdState &st,
                                       const NatOff &no) {
  x[0] = f32x16{};
  x[1] = f32x16{};
  bf16x8 a0 = lds_nat_o(bk, 0, 0, no), a1 = lds_nat_o(bk, 32, 0, no);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 n0 = a0, n1 = a1;
    if (ks + 1 < 8) {
      n0 = lds_nat_o(bk, 0, ks + 1, no);
      n1 = lds_nat_o(bk, 32, ks + 1, no);
    }
    __builtin_amdgcn_sched_barrier(0);
    x[0] = mfma32(a0, st.qreg[ks], x[0]);
    x[1] = mfma32(a1, st.qreg[ks], x[1]);
    a0 = n0;
    a1 = n1;
  }
}

// The same from an fp8 K tile and fp8 Q registers.
__device__ __forceinline__ void scores8(Scores &x, const u16 *bk, const FwdState &st,
                                        const Nat8Off &no) {
  x[0] = f32x16{};
  x[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    x[0] = mfma32_f8(lds_nat8(bk, 0, kk, no), st.q8[kk], x[0]);
    x[1] = mfma32_f8(lds_nat8(bk, 32, kk, no), st.q8[kk], x[1]);
  }
}

// Scores past the chunk's visible end or past this lane's causal bound get
// -inf. lim = last visible key of the block for this lane's half (relative
// to the block start, minus 4 hf).
__device__ __forceinline__ void mask_block(Scores &x, int lim) {
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    const int jj = 32 * (v >> 4) + 8 * ((v & 15) >> 2) + (v & 3);
    x[v >> 4][v & 15] = jj <= lim ? x[v >> 4][v & 15] : kNegInf;
  }
}

__device__ __forceinline__ float block_max(const Scores &x) {
  float m0 = fmaxf(fmaxf(x[0][0], x[0][1]), x[0][2]), m1 = fmaxf(fmaxf(x[1][0], x[1][1]), x[1][2]);
#pragma unroll
  for (int v = 3; v < 15; v += 2) {
    m0 = fmaxf(fmaxf(m0, x[0][v]), x[0][v + 1]);
    m1 = fmaxf(fmaxf(m1, x[1][v]), x[1][v + 1]);
  }
  m0 = fmaxf(m0, x[0][15]);
  m1 = fmaxf(m1, x[1][15]);
  return xhalf_max(fmaxf(m0, m1));
}

// P = exp2(c S - mu) packed to bf16, and its per-lane sum in fp32.
__device__ __forceinline__ float exp_block(bf16x8 (&pb)[4], const Scores &x, float c, float mu) {
  float psum = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = fast_exp2(fmaf(x[u >> 1][8 * (u & 1) + i], c, -mu));
      psum += e[i];
    }
    pb[u] = pack8(e);
  }
  return psum;
}

// O^T += V^T P^T.
__device__ __forceinline__ void pv_block(FwdState &st, const bf16x8 (&pb)[4], const u16 *bv,
                                         const TrOff &to) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.acc[dt] = mfma32(lds_tr_o(bv, 16 * u, dt, to), pb[u], st.acc[dt]);
}

constexpr int kWaves = 8;  // waves per workgroup, 32 query vectors each

// QK8: fp8 Q/K (else bf16); RUNS: walk the tile's run list (else the segments)
template <bool QK8, bool RUNS>
__global__ __launch_bounds__(kWaves * 64, 1) void fwd_ring_bf16_kernel(FwdRingArgs a) {
  // two K and two V tiles; separate objects so the LDS loads into one
  // buffer never order the reads of another
  __shared__ __attribute__((aligned(16))) u16 sK0[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sK1[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV0[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV1[kBN * kRS];
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
  const u16 *K = static_cast<const u16 *>(a.k);
  const u16 *V = static_cast<const u16 *>(a.v);
  const int bound = valid ? (t.src ? a.bound_branch[row] : a.bound_main[row]) : -1;

  FwdState st;
  if constexpr (QK8) {
    // fp8 rows are 128 bytes: this lane's bytes 64 kk + 32 hf .. + 31
    const char *qp = reinterpret_cast<const char *>(Q) + (int64_t(row) * a.hq + h) * 128 + hf * 32;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 lo = valid ? *reinterpret_cast<const u32x4 *>(qp + 64 * kk) : u32x4{0, 0, 0, 0};
      const u32x4 hi = valid ? *reinterpret_cast<const u32x4 *>(qp + 64 * kk + 16) : u32x4{0, 0, 0, 0};
      st.q8[kk] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                        int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
    }
  } else {
    const u16 *qp = Q + (int64_t(row) * a.hq + h) * 128 + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = valid ? *reinterpret_cast<const u32x4 *>(qp + ks * 16) : u32x4{0, 0, 0, 0};
      st.qreg[ks] = as_bf16x8(x);
    }
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.acc[dt] = f32x16{};
  st.mrun = 0.f;
  st.lsum = 0.f;
  const float c = a.scale_log2;
  const int64_t rs = int64_t(a.hkv) * 128;
  const int g = t.g;
  const int C = a.C, r = a.r, n_local = a.n_local;
  int nseg = 2 * C;  // end of the walk: segments, or runs

  const NatOff no = nat_offsets(lane);
  const Nat8Off no8 = nat8_offsets(lane);
  const TrOff to = tr_offsets(lane);
  const DmaOff<kWaves> dof =
      dma_offsets<kWaves>(wave, lane, [&](int rr) { return int64_t(rr) * rs; });
  // fp8 K: rows of hkv * 128 bytes
  const uint32_t dof8 = dma8_offset(wave, lane, rs);
  const char *K8 = reinterpret_cast<const char *>(a.k);
  auto rec = [&](const Blk &b) {
    BlkRec q;
    if (b.sg >= nseg) {
      q.off = 0;
      q.bytes = 0;
      q.lim = q.pos0 = q.need = 0;
      return q;
    }
    q.off = (b.s.krow + b.j0) * rs + g * 128;
    q.lim = min(kBN, b.s.n_hi - b.j0) - 1;
    q.bytes = uint32_t((q.lim * rs + 128) * 2);
    q.pos0 = b.s.cpos0 + b.j0;
    q.need = b.j0 + kBN > b.s.n_full;
    return q;
  };
  // rows of the block past the chunk's visible end are not read (their
  // scores are masked)
  auto load = [&](u16 *dk, u16 *dv, const BlkRec &q) {
    if constexpr (QK8) {
      // same rows at one byte per element: the element offset is the byte
      // offset, and the extent is half the bf16 one
      dma_tile64_f8(dk, buf_rsrc(K8 + q.off, q.bytes / 2), dof8, wave);
    } else {
      dma_tile64_buf<kWaves>(dk, buf_rsrc(K + q.off, q.bytes), dof, wave);
    }
    dma_tile64_buf<kWaves>(dv, buf_rsrc(V + q.off, q.bytes), dof, wave);
  };

  lds_zero(sK0, kBN * kRS, tid, kWaves * 64);
  lds_zero(sK1, kBN * kRS, tid, kWaves * 64);
  lds_zero(sV0, kBN * kRS, tid, kWaves * 64);
  lds_zero(sV1, kBN * kRS, tid, kWaves * 64);

  Blk wk;  // the walker: one block ahead of the one computed
  auto advance = [&]() {
    if constexpr (RUNS)
      next_run<kBN>(wk.sg, wk.j0, wk.s, sRuns, nseg);
    else
      next_block<kBN>(wk.sg, wk.j0, wk.s, t, C, r, n_local);
  };
  if constexpr (RUNS) {
    if (wave == 0) build_runs(sRuns, &sNRuns, t, C, r, n_local, lane);
    __syncthreads();
    nseg = uniform_int(sNRuns);
    first_run(wk.sg, wk.j0, wk.s, sRuns, nseg);
  } else {
    first_block<kBN>(wk.sg, wk.j0, wk.s, t, C, r, n_local);
  }
  BlkRec cur = rec(wk);
  if (cur.bytes) {  // else every row of the tile is a pad: O = 0, LSE = -inf
    advance();
    __syncthreads();  // LDS zeroed before any tile load lands
    load(sK0, sV0, cur);
    vm_wait<0>();
    bool first = true;
    // one block: KC/VC hold it, KN/VN receive the next one
    auto iter = [&](u16 *KC, u16 *VC, u16 *KN, u16 *VN) {
      __syncthreads();
      const BlkRec nxt = rec(wk);
      if (nxt.bytes) {
        load(KN, VN, nxt);
        advance();
      }
      if (wave_active) {
        Scores x;
        if constexpr (QK8)
          scores8(x, KC, st, no8);
        else
          scores(x, KC, st, no);
        if (cur.need) mask_block(x, min(cur.lim, bound - cur.pos0) - 4 * hf);
        if (first) {
          // every real row sees the first key of the first block
          const float bm = block_max(x) * c;
          st.mrun = (bm > kNegInf) ? bm : 0.f;
        }
        bf16x8 pb[4];
        float psum = exp_block(pb, x, c, st.mrun);
        if (__any(!(psum <= kOver))) {
          // a score rose far above the running max: raise it to the block's
          // exact max, rescale, redo the exponentials
          const float mnew = fmaxf(st.mrun, block_max(x) * c);
          const float alpha = fast_exp2(st.mrun - mnew);
          st.mrun = mnew;
          st.lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) st.acc[dt] *= alpha;
          psum = exp_block(pb, x, c, st.mrun);
        }
        st.lsum += psum;
        pv_block(st, pb, VC, to);
      }
      first = false;
      cur = nxt;
      vm_wait<0>();
    };
    while (true) {
      iter(sK0, sV0, sK1, sV1);
      if (!cur.bytes) break;
      iter(sK1, sV1, sK0, sV0);
      if (!cur.bytes) break;
    }
  }

  if (!valid) return;
  const float ltot = xhalf_sum(st.lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse = ltot > 0.f ? (st.mrun + log2f(ltot)) * kLn2 : kNegInf;
  const int64_t ob = (int64_t(row) * a.hq + h) * 128;
  if (t.src == 0) {
    u16 *O = static_cast<u16 *>(a.o);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * hf;
        u32x2 w;
        w.x = cvt_pk_bf16(st.acc[dt][4 * a4 + 0] * inv, st.acc[dt][4 * a4 + 1] * inv);
        w.y = cvt_pk_bf16(st.acc[dt][4 * a4 + 2] * inv, st.acc[dt][4 * a4 + 3] * inv);
        *reinterpret_cast<u32x2 *>(O + ob + d0) = w;
      }
    if (hf == 0) a.lse[int64_t(row) * a.hq + h] = lse;
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * hf;
        f32x4 w = {st.acc[dt][4 * a4 + 0] * inv, st.acc[dt][4 * a4 + 1] * inv,
                   st.acc[dt][4 * a4 + 2] * inv, st.acc[dt][4 * a4 + 3] * inv};
        *reinterpret_cast<f32x4 *>(a.om + ob + d0) = w;
      }
    if (hf == 0) a.lm[int64_t(row) * a.hq + h] = lse;
  }
}

// Every instance is instantiated explicitly: with only the implicit
// instantiation in the launchers, hipcc's host pass referenced the fp8
// instance's launch stub without emitting it.
template __global__ void fwd_ring_bf16_kernel<false, false>(FwdRingArgs);
template __global__ void fwd_ring_bf16_kernel<false, true>(FwdRingArgs);
template __global__ void fwd_ring_bf16_kernel<true, false>(FwdRingArgs);
template __global__ void fwd_ring_bf16_kernel<true, true>(FwdRingArgs);

}  // namespace

hipError_t launch_fwd_ring_bf16(const FwdRingArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (a.runs)
    hipLaunchKernelGGL((fwd_ring_bf16_kernel<false, true>), dim3(n_tiles), dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_ring_bf16_kernel<false, false>), dim3(n_tiles), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_ring_fp8(const FwdRingArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (a.runs)
    hipLaunchKernelGGL((fwd_ring_bf16_kernel<true, true>), dim3(n_tiles), dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_ring_bf16_kernel<true, false>), dim3(n_tiles), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
