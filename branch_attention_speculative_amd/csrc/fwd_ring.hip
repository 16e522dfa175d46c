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
// the score registers; V^T is read from the row-major V tile with the LDS
// transpose read, in the key order the score registers come in.
//
// Pipelining: K/V tiles are double-buffered in LDS and the next block is
// loaded straight from global memory into the idle buffer while the current
// one is computed (one barrier per block). The running max is only raised when a block's max exceeds it by
// more than 2^8 (in exp2 units), so most blocks skip the O rescale; the
// exponentials stay below 2^8 and the final normalisation uses the same max.

#include "kernels.h"
#include "ring_common.h"

namespace ba {

namespace {

constexpr int kBN = 64;          // keys per block
constexpr float kLazyMax = 8.f;  // rescale threshold (log2 units)

struct FwdState {
  bf16x8 qreg[8];
  f32x16 acc[4];
  float mrun, lsum;
};

// One 64-key block: scores, online softmax update, O += P V.
__device__ __forceinline__ void fwd_block(FwdState &st, const u16 *bk, const u16 *bv, const Seg &cs,
                                          int cj0, int bound, float c, int hf, const NatOff &no,
                                          const TrOff &to) {
  // S^T = K Q^T for 64 keys (two 32-key tiles)
  f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    s0 = mfma32(lds_nat_o(bk, 0, ks, no), st.qreg[ks], s0);
    s1 = mfma32(lds_nat_o(bk, 32, ks, no), st.qreg[ks], s1);
  }
  float x[32];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    x[v] = s0[v];
    x[16 + v] = s1[v];
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
  bmax = xhalf_max(bmax);
  const float cand = bmax * c;
  const bool up = cand > st.mrun + kLazyMax;
  if (__any(up)) {
    const float mnew = up ? cand : st.mrun;
    const float alpha = (mnew == st.mrun) ? 1.f : fast_exp2(st.mrun - mnew);
    st.mrun = mnew;
    st.lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.acc[dt] *= alpha;
  }
  const float mu = (st.mrun == kNegInf) ? 0.f : st.mrun;
  float psum = 0.f;
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    x[v] = fast_exp2(fmaf(x[v], c, -mu));
    psum += x[v];
  }
  st.lsum += psum;
  // O^T += V^T P^T
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bf16x8 pb = pack8(x + 8 * u);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.acc[dt] = mfma32(lds_tr_o(bv, 16 * u, dt, to), pb, st.acc[dt]);
  }
}

__global__ __launch_bounds__(256, 2) void fwd_ring_bf16_kernel(FwdRingArgs a) {
  // double-buffered K/V tiles; separate objects so the LDS loads into one
  // buffer never order the reads of the other
  __shared__ __attribute__((aligned(16))) u16 sK0[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV0[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sK1[kBN * kRS];
  __shared__ __attribute__((aligned(16))) u16 sV1[kBN * kRS];

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
  {
    const u16 *qp = Q + (int64_t(row) * a.hq + h) * 128 + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = valid ? *reinterpret_cast<const u32x4 *>(qp + ks * 16) : u32x4{0, 0, 0, 0};
      st.qreg[ks] = as_bf16x8(x);
    }
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.acc[dt] = f32x16{};
  st.mrun = kNegInf;
  st.lsum = 0.f;
  const float c = a.scale_log2;
  const int64_t rs = int64_t(a.hkv) * 128;
  const int g = t.g;

  const NatOff no = nat_offsets(lane);
  const TrOff to = tr_offsets(lane);
  const DmaOff<4> dof = dma_offsets<4>(wave, lane, [&](int r) { return int64_t(r) * rs; });
  // K/V rows j0 .. j0 + 63 of a chunk; rows past the chunk's visible end
  // are not read (their scores are masked)
  auto dma_kv = [&](const Seg &s, int j0, u16 *dk, u16 *dv) {
    const int64_t off = (s.krow + j0) * rs + g * 128;
    const uint32_t bytes = uint32_t(((min(kBN, s.n_hi - j0) - 1) * rs + 128) * 2);
    dma_tile64_buf<4>(dk, buf_rsrc(K + off, bytes), dof, wave);
    dma_tile64_buf<4>(dv, buf_rsrc(V + off, bytes), dof, wave);
  };

  lds_zero(sK0, kBN * kRS, tid, 256);
  lds_zero(sV0, kBN * kRS, tid, 256);
  lds_zero(sK1, kBN * kRS, tid, 256);
  lds_zero(sV1, kBN * kRS, tid, 256);
  __syncthreads();

  int sg, j0;
  Seg s;
  first_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
  const int nseg = 2 * a.C;
  if (sg < nseg) dma_kv(s, j0, sK0, sV0);
  dma_wait();
  __syncthreads();
  while (sg < nseg) {
    {
      const Seg cs = s;
      const int cj0 = j0;
      next_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
      if (sg < nseg) dma_kv(s, j0, sK1, sV1);
      if (wave_active) fwd_block(st, sK0, sV0, cs, cj0, bound, c, hf, no, to);
      dma_wait();
      __syncthreads();
    }
    if (sg >= nseg) break;
    {
      const Seg cs = s;
      const int cj0 = j0;
      next_block<kBN>(sg, j0, s, t, a.C, a.r, a.n_local);
      if (sg < nseg) dma_kv(s, j0, sK0, sV0);
      if (wave_active) fwd_block(st, sK1, sV1, cs, cj0, bound, c, hf, no, to);
      dma_wait();
      __syncthreads();
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

}  // namespace

hipError_t launch_fwd_ring_bf16(const FwdRingArgs &a, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_ring_bf16_kernel, dim3(n_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
