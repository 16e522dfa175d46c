// fp32 path of the ring part (forward, dQ, dK/dV) on the vector ALUs.
//
// Same visibility rules, ring order and outputs as the bf16 matrix-core
// kernels, with every value kept in fp32: one thread per query vector (row,
// q-head) for the forward and dQ, one thread per key vector (shard row,
// kv-head) for dK/dV. Each thread walks ring steps i = 0..C-1 over shard
// (r - i) mod C, head chunk then tail chunk (rainbus analysis of
// arXiv:2609.07108, method steps, steps two and five), carrying the
// online-softmax state across them.

#include "common.h"
#include "kernels.h"

namespace ba {

namespace {

// visible keys of a chunk for causal bound `bound`
__device__ __forceinline__ int chunk_visible(int bound, int cpos0, int c) {
  return min(max(bound - cpos0 + 1, 0), c);
}

template <int DIM>
__global__ __launch_bounds__(256) void fwd_ring_f32_kernel(FwdRingArgs a, F32Shape sh) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t(sh.n_local) + sh.n_branch) * sh.hq;
  if (gid >= total) return;
  const int64_t row_all = gid / sh.hq;
  const int h = int(gid % sh.hq);
  const int g = h / sh.G;
  const bool main = row_all < sh.n_local;
  const int64_t row = main ? row_all : row_all - sh.n_local;
  const int bound = main ? sh.bound_main[row] : sh.bound_branch[row];
  const int s = main ? sh.row_seq[row] : sh.branch_seq[row];
  const float *Q = static_cast<const float *>(main ? a.q : a.qb);
  const float *K = static_cast<const float *>(a.k);
  const float *V = static_cast<const float *>(a.v);
  const int64_t qh = row * sh.hq + h;
  float q[DIM], acc[DIM];
#pragma unroll
  for (int d = 0; d < DIM; ++d) {
    q[d] = Q[qh * DIM + d];
    acc[d] = 0.f;
  }
  float mrun = kNegInf, lsum = 0.f;
  if (bound >= 0) {
    const int c = sh.chunk[s], off = sh.cu_local[s];
    for (int i = 0; i < sh.C; ++i) {
      int shard = sh.r - i;
      if (shard < 0) shard += sh.C;
      for (int half = 0; half < 2; ++half) {
        const int chunk = half ? 2 * sh.C - 1 - shard : shard;
        const int nvis = chunk_visible(bound, chunk * c, c);
        const int64_t krow0 = int64_t(shard) * sh.n_local + off + int64_t(half) * c;
        for (int jj = 0; jj < nvis; ++jj) {
          const int64_t ko = ((krow0 + jj) * sh.hkv + g) * DIM;
          float x = 0.f;
#pragma unroll
          for (int d = 0; d < DIM; ++d) x = fmaf(q[d], K[ko + d], x);
          x *= sh.scale_log2;
          const float mnew = fmaxf(mrun, x);
          const float alpha = exp2f(mrun - mnew);
          const float p = exp2f(x - mnew);
          lsum = lsum * alpha + p;
#pragma unroll
          for (int d = 0; d < DIM; ++d) acc[d] = fmaf(p, V[ko + d], acc[d] * alpha);
          mrun = mnew;
        }
      }
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float lse = lsum > 0.f ? (mrun + log2f(lsum)) * kLn2 : kNegInf;
  if (main) {
    float *O = static_cast<float *>(a.o);
#pragma unroll
    for (int d = 0; d < DIM; ++d) O[qh * DIM + d] = acc[d] * inv;
    a.lse[qh] = lse;
  } else {
#pragma unroll
    for (int d = 0; d < DIM; ++d) a.om[qh * DIM + d] = acc[d] * inv;
    a.lm[qh] = lse;
  }
}

template <int DIM>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdDqArgs a, F32Shape sh) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t(sh.n_local) + sh.n_branch) * sh.hq;
  if (gid >= total) return;
  const int64_t row_all = gid / sh.hq;
  const int h = int(gid % sh.hq);
  const int g = h / sh.G;
  const bool main = row_all < sh.n_local;
  const int64_t row = main ? row_all : row_all - sh.n_local;
  const int bound = main ? sh.bound_main[row] : sh.bound_branch[row];
  const int s = main ? sh.row_seq[row] : sh.branch_seq[row];
  const float *Q = static_cast<const float *>(main ? a.q : a.qb);
  const float *DO = static_cast<const float *>(main ? a.dout : a.doutb);
  const float *K = static_cast<const float *>(a.k);
  const float *V = static_cast<const float *>(a.v);
  const int64_t qh = row * sh.hq + h;
  float dq[DIM];
#pragma unroll
  for (int d = 0; d < DIM; ++d) dq[d] = 0.f;
  if (bound >= 0) {
    const float lse2 = (main ? a.lse[qh] : a.lseb[qh]) * kLog2e;
    const float ndel = a.ndelta[gid];
    const int c = sh.chunk[s], off = sh.cu_local[s];
    for (int i = 0; i < sh.C; ++i) {
      int shard = sh.r - i;
      if (shard < 0) shard += sh.C;
      for (int half = 0; half < 2; ++half) {
        const int chunk = half ? 2 * sh.C - 1 - shard : shard;
        const int nvis = chunk_visible(bound, chunk * c, c);
        const int64_t krow0 = int64_t(shard) * sh.n_local + off + int64_t(half) * c;
        for (int jj = 0; jj < nvis; ++jj) {
          const int64_t ko = ((krow0 + jj) * sh.hkv + g) * DIM;
          float x = 0.f, dp = 0.f;
          for (int d = 0; d < DIM; ++d) {
            x = fmaf(Q[qh * DIM + d], K[ko + d], x);
            dp = fmaf(DO[qh * DIM + d], V[ko + d], dp);
          }
          const float p = exp2f(x * sh.scale_log2 - lse2);
          const float ds = p * (dp + ndel);
#pragma unroll
          for (int d = 0; d < DIM; ++d) dq[d] = fmaf(ds, K[ko + d], dq[d]);
        }
      }
    }
  }
  float *DQ = static_cast<float *>(main ? a.dq : a.dqb);
#pragma unroll
  for (int d = 0; d < DIM; ++d) {
    float x = dq[d] * sh.scale;
    if (!main) x += a.dq_local[qh * DIM + d];
    DQ[qh * DIM + d] = x;
  }
}

// one thread per (key row of a shard, kv-head): walk every local query row
// (main rows, then branch rows) of the key's sequence whose bound reaches it
template <int DIM>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(BwdDkdvArgs a, F32Shape sh) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(sh.C) * sh.n_local * sh.hkv;
  if (gid >= total) return;
  const int64_t krow = gid / sh.hkv;
  const int g = int(gid % sh.hkv);
  const int shard = int(krow / sh.n_local);
  const int i = int(krow % sh.n_local);
  const int s = sh.row_seq[i];  // every shard shares the per-sequence row layout
  const int c = sh.chunk[s];
  const int ii = i - sh.cu_local[s];
  const int half = ii >= c ? 1 : 0;
  const int chunk = half ? 2 * sh.C - 1 - shard : shard;
  const int kpos = chunk * c + (ii - half * c);
  const float *K = static_cast<const float *>(a.k);
  const float *V = static_cast<const float *>(a.v);
  const int64_t ko = gid * DIM;
  float dk[DIM], dv[DIM];
#pragma unroll
  for (int d = 0; d < DIM; ++d) dk[d] = dv[d] = 0.f;
  if (kpos < sh.seq_len[s]) {
    for (int src = 0; src < 2; ++src) {
      const float *Q = static_cast<const float *>(src ? a.qb : a.q);
      const float *DO = static_cast<const float *>(src ? a.doutb : a.dout);
      const float *LSE = src ? a.lseb : a.lse;
      const int32_t *BOUND = src ? sh.bound_branch : sh.bound_main;
      const float *NDEL = a.ndelta + (src ? int64_t(sh.n_local) * sh.hq : 0);
      const int lo = src ? sh.branch_off[sh.seq_a0[s]] : sh.cu_local[s];
      const int hi = src ? sh.branch_off[sh.seq_a0[s + 1]] : sh.cu_local[s + 1];
      for (int q = lo; q < hi; ++q) {
        if (BOUND[q] < kpos) continue;
        for (int hh = 0; hh < sh.G; ++hh) {
          const int64_t qh = int64_t(q) * sh.hq + g * sh.G + hh;
          float x = 0.f, dp = 0.f;
          for (int d = 0; d < DIM; ++d) {
            x = fmaf(Q[qh * DIM + d], K[ko + d], x);
            dp = fmaf(DO[qh * DIM + d], V[ko + d], dp);
          }
          const float p = exp2f(x * sh.scale_log2 - LSE[qh] * kLog2e);
          const float ds = p * (dp + NDEL[qh]);
#pragma unroll
          for (int d = 0; d < DIM; ++d) {
            dk[d] = fmaf(ds, Q[qh * DIM + d], dk[d]);
            dv[d] = fmaf(p, DO[qh * DIM + d], dv[d]);
          }
        }
      }
    }
  }
  float *DK = static_cast<float *>(a.dk);
  float *DV = static_cast<float *>(a.dv);
#pragma unroll
  for (int d = 0; d < DIM; ++d) {
    DK[ko + d] = dk[d] * sh.scale;
    DV[ko + d] = dv[d];
  }
}

int64_t blocks_for(int64_t n) { return (n + 255) / 256; }

}  // namespace

hipError_t launch_fwd_ring_f32(const FwdRingArgs &a, const F32Shape &sh, hipStream_t s) {
  const int64_t nb = blocks_for((int64_t(sh.n_local) + sh.n_branch) * sh.hq);
  if (nb <= 0) return hipSuccess;
  if (sh.d == 64)
    hipLaunchKernelGGL(fwd_ring_f32_kernel<64>, dim3(nb), dim3(256), 0, s, a, sh);
  else
    hipLaunchKernelGGL(fwd_ring_f32_kernel<128>, dim3(nb), dim3(256), 0, s, a, sh);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const BwdDqArgs &a, const F32Shape &sh, hipStream_t s) {
  const int64_t nb = blocks_for((int64_t(sh.n_local) + sh.n_branch) * sh.hq);
  if (nb <= 0) return hipSuccess;
  if (sh.d == 64)
    hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3(nb), dim3(256), 0, s, a, sh);
  else
    hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, dim3(nb), dim3(256), 0, s, a, sh);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const BwdDkdvArgs &a, const F32Shape &sh, hipStream_t s) {
  const int64_t nb = blocks_for(int64_t(sh.C) * sh.n_local * sh.hkv);
  if (nb <= 0) return hipSuccess;
  if (sh.d == 64)
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, dim3(nb), dim3(256), 0, s, a, sh);
  else
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, dim3(nb), dim3(256), 0, s, a, sh);
  return hipGetLastError();
}

}  // namespace ba
