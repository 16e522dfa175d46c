// Rank-local branch attention (forward partial + Eq. 2 merge, backward) and
// the backward preprocess Delta = rowsum(dO * O) (with LSE * log2(e) for the
// ring replay).
//
// The branch part is small and stays on the rank that owns the anchor, with
// no communication (ai.info summary, Key Contributions 1 and Methodology).
// Each branch row j of an anchor sees that anchor's branch keys j' <= j (TTT
// chains, causal blocks) or all of them (bidirectional blocks). Its partial
// (O_b, l_b) is merged with the main-sequence partial (O_m, l_m) produced by
// the ring kernel using the online-softmax rule (rainbus analysis, core
// method, Eq. 2): l = log(e^lm + e^lb), O = (e^(lm-l) O_m + e^(lb-l) O_b) /
// (e^(lm-l) + e^(lb-l)).
//
// These kernels run on the vector ALUs: a branch holds at most 64 keys, so
// the work is tiny next to the ring part. Templated on element type (bf16
// bits or float), head dim and the longest branch of the plan.

#include "common.h"
#include "kernels.h"

namespace ba {

namespace {

template <typename T>
__device__ __forceinline__ float ldf(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ldf<u16>(const u16 *p, int64_t i) {
  return bf2f(p[i]);
}
template <>
__device__ __forceinline__ float ldf<float>(const float *p, int64_t i) {
  return p[i];
}

// load 8 consecutive elements as floats (16-byte aligned for bf16, 32 for fp32)
template <typename T>
__device__ __forceinline__ void ld8(const T *p, int64_t i, float (&o)[8]);
template <>
__device__ __forceinline__ void ld8<u16>(const u16 *p, int64_t i, float (&o)[8]) {
  const u32x4 x = *reinterpret_cast<const u32x4 *>(p + i);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(x[k] << 16);
    o[2 * k + 1] = __uint_as_float(x[k] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void ld8<float>(const float *p, int64_t i, float (&o)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p + i);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + i + 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = a[k];
    o[4 + k] = b[k];
  }
}

// fp8 E4M3 codes (Q and K of the fp8 path): 8 consecutive bytes, 8-byte aligned
template <>
__device__ __forceinline__ void ld8<uint8_t>(const uint8_t *p, int64_t i, float (&o)[8]) {
  const u32x2 x = *reinterpret_cast<const u32x2 *>(p + i);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(x[k]), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(x[k]), true);
    o[4 * k] = lo[0];
    o[4 * k + 1] = lo[1];
    o[4 * k + 2] = hi[0];
    o[4 * k + 3] = hi[1];
  }
}

// load 4 consecutive elements as floats (8-byte aligned for bf16, 16 for fp32)
template <typename T>
__device__ __forceinline__ void ld4(const T *p, int64_t i, float (&o)[4]);
template <>
__device__ __forceinline__ void ld4<u16>(const u16 *p, int64_t i, float (&o)[4]) {
  const u32x2 x = *reinterpret_cast<const u32x2 *>(p + i);
  o[0] = __uint_as_float(x.x << 16);
  o[1] = __uint_as_float(x.x & 0xffff0000u);
  o[2] = __uint_as_float(x.y << 16);
  o[3] = __uint_as_float(x.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void ld4<float>(const float *p, int64_t i, float (&o)[4]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p + i);
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = a[k];
}

// 8 consecutive elements as loaded (raw), and their conversion to floats: the
// kernels issue every global load of a query vector before the arithmetic
// that uses the first one, so that the loads' latencies overlap
template <typename T>
struct Raw8;
template <>
struct Raw8<u16> {
  u32x4 x;
};
template <>
struct Raw8<float> {
  f32x4 a, b;
};
template <>
struct Raw8<uint8_t> {
  u32x2 x;
};
template <typename T>
__device__ __forceinline__ Raw8<T> ldraw8(const T *p, int64_t i);
template <>
__device__ __forceinline__ Raw8<u16> ldraw8<u16>(const u16 *p, int64_t i) {
  return {*reinterpret_cast<const u32x4 *>(p + i)};
}
template <>
__device__ __forceinline__ Raw8<float> ldraw8<float>(const float *p, int64_t i) {
  return {*reinterpret_cast<const f32x4 *>(p + i), *reinterpret_cast<const f32x4 *>(p + i + 4)};
}
template <>
__device__ __forceinline__ Raw8<uint8_t> ldraw8<uint8_t>(const uint8_t *p, int64_t i) {
  return {*reinterpret_cast<const u32x2 *>(p + i)};
}
__device__ __forceinline__ void cvt8(const Raw8<u16> &r, float (&o)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(r.x[k] << 16);
    o[2 * k + 1] = __uint_as_float(r.x[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void cvt8(const Raw8<float> &r, float (&o)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = r.a[k];
    o[4 + k] = r.b[k];
  }
}
__device__ __forceinline__ void cvt8(const Raw8<uint8_t> &r, float (&o)[8]) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(r.x[k]), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(r.x[k]), true);
    o[4 * k] = lo[0];
    o[4 * k + 1] = lo[1];
    o[4 * k + 2] = hi[0];
    o[4 * k + 3] = hi[1];
  }
}
// a raw copy into LDS (8 elements at lds, 16-byte aligned)
__device__ __forceinline__ void keep8(const Raw8<u16> &r, u16 *lds) {
  *reinterpret_cast<u32x4 *>(lds) = r.x;
}
__device__ __forceinline__ void keep8(const Raw8<float> &r, float *lds) {
  *reinterpret_cast<f32x4 *>(lds) = r.a;
  *reinterpret_cast<f32x4 *>(lds + 4) = r.b;
}

template <typename T>
__device__ __forceinline__ void st8(T *p, int64_t i, const float (&v)[8]);
template <>
__device__ __forceinline__ void st8<u16>(u16 *p, int64_t i, const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = pack_bf2(v[2 * k], v[2 * k + 1]);
  *reinterpret_cast<u32x4 *>(p + i) = w;
}
template <>
__device__ __forceinline__ void st8<float>(float *p, int64_t i, const float (&v)[8]) {
  *reinterpret_cast<f32x4 *>(p + i) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4 *>(p + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Stage branch key or value rows of a tile (rows [base, base + rows), kv-head
// g) in LDS in their input type, row-major [row][DIM] (half the LDS of floats
// for bf16, a quarter for fp8, so that more workgroups fit on a compute unit).
template <typename T, int DIM>
__device__ __forceinline__ void stage_rows(const T *X, int base, int rows, int g, int hkv, T *sX) {
  constexpr int PER = 16 / sizeof(T);  // elements per 16-byte chunk
  for (int id = threadIdx.x; id < rows * (DIM / PER); id += blockDim.x) {
    const int rr = id / (DIM / PER), dc = id % (DIM / PER);
    const int64_t off = (int64_t(base + rr) * hkv + g) * DIM + dc * PER;
    *reinterpret_cast<u32x4 *>(sX + rr * DIM + dc * PER) = *reinterpret_cast<const u32x4 *>(X + off);
  }
}
template <typename T, int DIM>
__device__ __forceinline__ void stage_branch_kv(const T *KB, const T *VB, int base, int rows,
                                                int g, int hkv, T *sK, T *sV) {
  stage_rows<T, DIM>(KB, base, rows, g, hkv, sK);
  stage_rows<T, DIM>(VB, base, rows, g, hkv, sV);
}

// ---------------------------------------------------------------------------

// TQ: element type of qb and kb; T: of vb and ob.
template <typename TQ, typename T, int DIM, int MAXB>
__global__ __launch_bounds__(256) void fwd_branch_kernel(FwdBranchArgs a) {
  __shared__ __attribute__((aligned(16))) TQ sK[kMaxBranch * DIM];
  __shared__ __attribute__((aligned(16))) T sV[kMaxBranch * DIM];
  const BTile t = a.btiles[blockIdx.x];
  if (t.rows == 0) return;
  const int base = a.branch_off[t.a0];
  const int G = a.G;
  const TQ *QB = static_cast<const TQ *>(a.qb);
  stage_rows<TQ, DIM>(static_cast<const TQ *>(a.kb), base, t.rows, t.g, a.hkv, sK);
  stage_rows<T, DIM>(static_cast<const T *>(a.vb), base, t.rows, t.g, a.hkv, sV);
  __syncthreads();
  // four threads per query vector, each over a quarter of D: contiguous
  // reads of q and of the partial, contiguous writes of the output
  const int ql = threadIdx.x >> 2, sub = threadIdx.x & 3;
  constexpr int QD = DIM / 4;
  for (int qv = ql; qv < t.rows * G; qv += blockDim.x / 4) {  // uniform per group of four
    const int row = base + qv / G;
    const int h = t.g * G + qv % G;
    const int an = a.b_anchor[row];
    const int lo = a.branch_off[an];
    const int n = a.branch_off[an + 1] - lo;
    const int j = row - lo;
    const int nvis = a.bidir ? n : j + 1;
    const int kl0 = lo - base;
    const int64_t qh = int64_t(row) * a.hq + h;
    Raw8<TQ> qr[QD / 8];
    Raw8<float> mr[QD / 8];
#pragma unroll
    for (int dc = 0; dc < QD / 8; ++dc) qr[dc] = ldraw8<TQ>(QB, qh * DIM + sub * QD + dc * 8);
#pragma unroll
    for (int dc = 0; dc < QD / 8; ++dc) mr[dc] = ldraw8<float>(a.om, qh * DIM + sub * QD + dc * 8);
    const float lm2 = a.lm[qh] * kLog2e;  // main-sequence LSE (log2)
    float s[MAXB];
#pragma unroll
    for (int jj = 0; jj < MAXB; ++jj) s[jj] = 0.f;
#pragma unroll
    for (int dc = 0; dc < QD / 8; ++dc) {
      const int d0 = sub * QD + dc * 8;
      float q8[8];
      cvt8(qr[dc], q8);
#pragma unroll
      for (int jj = 0; jj < MAXB; ++jj) {
        if (jj < nvis) {
          float kr[8];
          ld8<TQ>(sK, (kl0 + jj) * DIM + d0, kr);
          float acc = s[jj];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(q8[e], kr[e], acc);
          s[jj] = acc;
        }
      }
    }
    // full dot products: sum over the four quarters
#pragma unroll
    for (int jj = 0; jj < MAXB; ++jj) {
      s[jj] += __shfl_xor(s[jj], 1, 4);
      s[jj] += __shfl_xor(s[jj], 2, 4);
    }
    // branch partial: max and sum in the log2 domain
    float mb = kNegInf;
#pragma unroll
    for (int jj = 0; jj < MAXB; ++jj)
      if (jj < nvis) {
        s[jj] *= a.scale_log2;
        mb = fmaxf(mb, s[jj]);
      }
    float lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < MAXB; ++jj) {
      s[jj] = jj < nvis ? fast_exp2(s[jj] - mb) : 0.f;
      lsum += s[jj];
    }
    const float lb2 = mb + log2f(lsum);  // branch-local LSE (log2)
    // Eq. 2: l = log(e^lm + e^lb); weights e^(lm - l), e^(lb - l)
    const float hi = fmaxf(lm2, lb2);
    const float l2 = hi + log2f(fast_exp2(lm2 - hi) + fast_exp2(lb2 - hi));
    const float wm = fast_exp2(lm2 - l2);
    const float wb = fast_exp2(lb2 - l2);
    const float norm = 1.f / (wm + wb);
    const float cm = wm * norm, cb = wb * norm / lsum;
    T *OB = static_cast<T *>(a.ob);
#pragma unroll
    for (int dc = 0; dc < QD / 8; ++dc) {
      const int d0 = sub * QD + dc * 8;
      float o8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = 0.f;
#pragma unroll
      for (int jj = 0; jj < MAXB; ++jj) {
        if (jj < nvis) {
          float vr[8];
          ld8<T>(sV, (kl0 + jj) * DIM + d0, vr);
#pragma unroll
          for (int e = 0; e < 8; ++e) o8[e] = fmaf(s[jj], vr[e], o8[e]);
        }
      }
      float m8[8];
      cvt8(mr[dc], m8);
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = cm * m8[e] + cb * o8[e];
      st8<T>(OB, qh * DIM + d0, o8);
    }
    if (sub == 0) a.lseb[qh] = l2 * kLn2;
  }
}

// ---------------------------------------------------------------------------

template <typename T, int DIM>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdPreArgs a) {
  // 16 lanes per (row, head); rows are main rows then branch rows
  const int64_t pair = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int64_t total = (int64_t(a.n_local) + a.n_branch) * a.hq;
  float acc = 0.f;
  bool pad = true;
  float l2 = 0.f;
  if (pair < total) {
    const int64_t row = pair / a.hq;
    const bool main = row < a.n_local;
    pad = main && a.bound_main[row] < 0;
    const int64_t qh = main ? pair : pair - int64_t(a.n_local) * a.hq;
    l2 = (main ? a.lse : a.lseb)[qh] * kLog2e;
    const T *O = static_cast<const T *>(main ? a.o : a.ob);
    const T *DO = static_cast<const T *>(main ? a.dout : a.doutb);
    constexpr int PER = DIM / 16;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int64_t i = qh * DIM + sub * PER + e;
      acc = fmaf(ldf<T>(O, i), ldf<T>(DO, i), acc);
    }
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (pair < total && sub == 0) {
    a.ndelta[pair] = pad ? 0.f : -acc;
    a.lse2[pair] = pad ? 0.f : l2;
  }
}

// ---------------------------------------------------------------------------

constexpr int kBQ = 64;  // query vectors per backward chunk (four threads each)

template <typename T, int DIM, int MAXB>
__global__ __launch_bounds__(256) void bwd_branch_kernel(BwdBranchArgs a) {
  // K / V in the input type; P and dS of each query vector of a chunk against
  // the keys of its own anchor (index 0 = the anchor's first key)
  __shared__ __attribute__((aligned(16))) T sK[kMaxBranch * DIM];
  __shared__ __attribute__((aligned(16))) T sV[kMaxBranch * DIM];
  __shared__ float sP[kBQ * MAXB];
  __shared__ float sS[kBQ * MAXB];
  // q and dO of the chunk's query vectors, kept from phase 1 for phase 2
  __shared__ __attribute__((aligned(16))) T sQ[kBQ * DIM];
  __shared__ __attribute__((aligned(16))) T sDO[kBQ * DIM];
  const BTile t = a.btiles[blockIdx.x];
  if (t.rows == 0) return;
  const int base = a.branch_off[t.a0];
  const int G = a.G;
  const int tid = threadIdx.x;
  const T *QB = static_cast<const T *>(a.qb);
  const T *DOB = static_cast<const T *>(a.doutb);
  stage_branch_kv<T, DIM>(static_cast<const T *>(a.kb), static_cast<const T *>(a.vb), base, t.rows,
                          t.g, a.hkv, sK, sV);
  // phase-2 items: (key row kl, 8 consecutive d) -> fixed per thread
  constexpr int ITEMS = (kMaxBranch * DIM / 8 + 255) / 256;
  float adk[ITEMS][8], adv[ITEMS][8];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it)
#pragma unroll
    for (int e = 0; e < 8; ++e) adk[it][e] = adv[it][e] = 0.f;
  // each phase-2 item's key row and the range of its anchor's rows, fixed
  // over the chunks
  // (rows past the tile read the tile's last row; such items are skipped)
  int it_lo[ITEMS], it_hi[ITEMS], it_an[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it)
    it_an[it] = a.b_anchor[base + min((tid + 256 * it) / (DIM / 8), t.rows - 1)];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    it_lo[it] = a.branch_off[it_an[it]] - base;
    it_hi[it] = a.branch_off[it_an[it] + 1] - base;
  }
  const int nqv = t.rows * G;
  // phase 1: four threads per query vector of the chunk, each over a quarter of D
  const int ql = tid >> 2, sub = tid & 3;
  constexpr int QD = DIM / 4;  // dims per thread
  for (int c0 = 0; c0 < nqv; c0 += kBQ) {
    const int nq = min(kBQ, nqv - c0);
    __syncthreads();  // staged K/V visible; previous chunk's sP/sS reads done
    if (ql < nq) {  // uniform over each group of four
      const int qv = c0 + ql;
      const int row = base + qv / G;
      const int h = t.g * G + qv % G;
      const int an = a.b_anchor[row];
      const int lo = a.branch_off[an];
      const int n = a.branch_off[an + 1] - lo;
      const int j = row - lo;
      const int nvis = a.bidir ? n : j + 1;
      const int kl0 = lo - base;
      const int64_t qh = int64_t(row) * a.hq + h;
      Raw8<T> qr[QD / 8], dr[QD / 8];
#pragma unroll
      for (int dc = 0; dc < QD / 8; ++dc) {
        qr[dc] = ldraw8<T>(QB, qh * DIM + sub * QD + dc * 8);
        dr[dc] = ldraw8<T>(DOB, qh * DIM + sub * QD + dc * 8);
      }
      const float lse2 = a.lseb[qh] * kLog2e;
      const float ndel = a.ndelta_b[qh];
      float s[MAXB], dp[MAXB];
#pragma unroll
      for (int jj = 0; jj < MAXB; ++jj) s[jj] = dp[jj] = 0.f;
#pragma unroll
      for (int dc = 0; dc < QD / 8; ++dc) {
        const int d0 = sub * QD + dc * 8;
        float q8[8], d8[8];
        keep8(qr[dc], sQ + ql * DIM + d0);
        keep8(dr[dc], sDO + ql * DIM + d0);
        cvt8(qr[dc], q8);
        cvt8(dr[dc], d8);
#pragma unroll
        for (int jj = 0; jj < MAXB; ++jj) {
          if (jj < nvis) {
            float kr[8], vr[8];
            ld8<T>(sK, (kl0 + jj) * DIM + d0, kr);
            ld8<T>(sV, (kl0 + jj) * DIM + d0, vr);
            float as = s[jj], ad = dp[jj];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              as = fmaf(q8[e], kr[e], as);
              ad = fmaf(d8[e], vr[e], ad);
            }
            s[jj] = as;
            dp[jj] = ad;
          }
        }
      }
      // full dot products: sum over the four quarters
#pragma unroll
      for (int jj = 0; jj < MAXB; ++jj) {
        s[jj] += __shfl_xor(s[jj], 1, 4);
        s[jj] += __shfl_xor(s[jj], 2, 4);
        dp[jj] += __shfl_xor(dp[jj], 1, 4);
        dp[jj] += __shfl_xor(dp[jj], 2, 4);
      }
#pragma unroll
      for (int jj = 0; jj < MAXB; ++jj) {
        float p = 0.f, d = 0.f;
        if (jj < nvis) {
          p = fast_exp2(s[jj] * a.scale_log2 - lse2);
          d = p * (dp[jj] + ndel);
        }
        s[jj] = d;  // keep dS for the dQ sum
        if (sub == 0) {
          sP[ql * MAXB + jj] = p;
          sS[ql * MAXB + jj] = d;
        }
      }
      // this thread's quarter of the branch-key share of dQ
#pragma unroll
      for (int dc = 0; dc < QD / 8; ++dc) {
        const int d0 = sub * QD + dc * 8;
        float o8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = 0.f;
#pragma unroll
        for (int jj = 0; jj < MAXB; ++jj) {
          if (jj < nvis) {
            float kr[8];
            ld8<T>(sK, (kl0 + jj) * DIM + d0, kr);
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = fmaf(s[jj], kr[e], o8[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] *= a.scale;
        st8<float>(a.dq_local, qh * DIM + d0, o8);
      }
    }
    __syncthreads();
    // phase 2: dK[kl] += scale * sum_q dS[q][kl] Q[q]; dV[kl] += sum_q P[q][kl] dO[q]
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + 256 * it;
      if (item < t.rows * (DIM / 8)) {
        const int kl = item / (DIM / 8), d4 = item % (DIM / 8);
        const int lo = it_lo[it], hi = it_hi[it];
        const int q_lo = max(lo * G, c0), q_hi = min(hi * G, c0 + nq);
        // this key is entry kl - lo of its anchor's queries' P / dS rows
        for (int qv = q_lo; qv < q_hi; ++qv) {
          const float p = sP[(qv - c0) * MAXB + kl - lo];
          const float d = sS[(qv - c0) * MAXB + kl - lo];
          if (p == 0.f && d == 0.f) continue;
          float q4[8], o4[8];
          ld8<T>(sQ, (qv - c0) * DIM + d4 * 8, q4);
          ld8<T>(sDO, (qv - c0) * DIM + d4 * 8, o4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            adk[it][e] = fmaf(d, q4[e], adk[it][e]);
            adv[it][e] = fmaf(p, o4[e], adv[it][e]);
          }
        }
      }
    }
  }
  T *DKB = static_cast<T *>(a.dkb);
  T *DVB = static_cast<T *>(a.dvb);
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int item = tid + 256 * it;
    if (item < t.rows * (DIM / 8)) {
      const int kl = item / (DIM / 8), d4 = item % (DIM / 8);
      const int64_t off = (int64_t(base + kl) * a.hkv + t.g) * DIM + d4 * 8;
      float k8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) k8[e] = adk[it][e] * a.scale;
      st8<T>(DKB, off, k8);
      st8<T>(DVB, off, adv[it]);
    }
  }
}

// E4M3 codes to bf16, 8 per thread. Every E4M3 value (NaN included) is a
// bf16 value: the fp32 decode has zeros in its low 16 bits, so keeping the
// high half is exact.
__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint8_t *in, u16 *out, int64_t n8) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  cvt8(ldraw8<uint8_t>(in, i * 8), v);
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xffff0000u);
  *reinterpret_cast<u32x4 *>(out + i * 8) = w;
}

template <typename TQ, typename T, int DIM>
hipError_t fwd_branch_dispatch(const FwdBranchArgs &a, int n, int maxb, hipStream_t s) {
  if (maxb <= 8)
    hipLaunchKernelGGL((fwd_branch_kernel<TQ, T, DIM, 8>), dim3(n), dim3(256), 0, s, a);
  else if (maxb <= 16)
    hipLaunchKernelGGL((fwd_branch_kernel<TQ, T, DIM, 16>), dim3(n), dim3(256), 0, s, a);
  else if (maxb <= 32)
    hipLaunchKernelGGL((fwd_branch_kernel<TQ, T, DIM, 32>), dim3(n), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_branch_kernel<TQ, T, DIM, 64>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DIM>
hipError_t bwd_branch_dispatch(const BwdBranchArgs &a, int n, int maxb, hipStream_t s) {
  if (maxb <= 8)
    hipLaunchKernelGGL((bwd_branch_kernel<T, DIM, 8>), dim3(n), dim3(256), 0, s, a);
  else if (maxb <= 16)
    hipLaunchKernelGGL((bwd_branch_kernel<T, DIM, 16>), dim3(n), dim3(256), 0, s, a);
  else if (maxb <= 32)
    hipLaunchKernelGGL((bwd_branch_kernel<T, DIM, 32>), dim3(n), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_branch_kernel<T, DIM, 64>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_branch(const FwdBranchArgs &a, int n_tiles, int dtype, int maxb,
                             hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (dtype == BA_BF16) return fwd_branch_dispatch<u16, u16, 128>(a, n_tiles, maxb, s);
  if (dtype == BA_FP8) return fwd_branch_dispatch<uint8_t, u16, 128>(a, n_tiles, maxb, s);
  if (a.d == 64) return fwd_branch_dispatch<float, float, 64>(a, n_tiles, maxb, s);
  return fwd_branch_dispatch<float, float, 128>(a, n_tiles, maxb, s);
}

hipError_t launch_bwd_pre(const BwdPreArgs &a, int dtype, hipStream_t s) {
  const int64_t total = (int64_t(a.n_local) + a.n_branch) * a.hq;
  const int64_t blocks = (total + 15) / 16;
  if (blocks <= 0) return hipSuccess;
  if (dtype == BA_BF16)
    hipLaunchKernelGGL((bwd_pre_kernel<u16, 128>), dim3(blocks), dim3(256), 0, s, a);
  else if (a.d == 64)
    hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fp8_to_bf16(const uint8_t *in, uint16_t *out, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3(uint32_t(blocks)), dim3(256), 0, s, in, out, n8);
  return hipGetLastError();
}

hipError_t launch_bwd_branch(const BwdBranchArgs &a, int n_tiles, int dtype, int maxb,
                             hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  if (dtype == BA_BF16) return bwd_branch_dispatch<u16, 128>(a, n_tiles, maxb, s);
  if (a.d == 64) return bwd_branch_dispatch<float, 64>(a, n_tiles, maxb, s);
  return bwd_branch_dispatch<float, 128>(a, n_tiles, maxb, s);
}

}  // namespace ba
