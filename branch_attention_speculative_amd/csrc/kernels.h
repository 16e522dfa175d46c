// Kernel argument blocks and launcher declarations (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace ba {

constexpr float kLog2eHost = 1.4426950408889634f;

// Ring-step forward over the main keys of every shard (the causal main
// sequence part), for main rows and for the main prefix of branch rows.
struct FwdRingArgs {
  const void *q, *qb, *k, *v;
  void *o;          // main rows: final output (no branch part)
  float *lse;       // main rows: final LSE (natural log)
  float *om;        // branch rows: main partial O_m, fp32, normalised
  float *lm;        // branch rows: main partial LSE
  const QTile *qtiles;
  const int32_t *bound_main, *bound_branch;
  int32_t n_local, n_branch, hq, hkv, G, log2G, C, r, d;
  float scale_log2;  // softmax scale * log2(e)
  float scale;
  int32_t runs;      // walk each tile's run list (short chunks) instead of its segments
};

// Branch-local forward and the Eq. 2 merge with the main partial.
struct FwdBranchArgs {
  const void *qb, *kb, *vb;
  const float *om, *lm;
  void *ob;
  float *lseb;
  const BTile *btiles;
  const int32_t *branch_off, *b_anchor;
  int32_t hq, hkv, G, d, bidir;
  float scale_log2;
};

// -Delta = -rowsum(dO * O) for main rows then branch rows (stored negated:
// the kernels that use it accumulate dP onto it).
struct BwdPreArgs {
  const void *o, *ob, *dout, *doutb;
  const float *lse, *lseb;
  const int32_t *bound_main;
  float *ndelta;  // [(N + NB) * hq]
  float *lse2;   // [(N + NB) * hq]: LSE * log2(e)
  int32_t n_local, n_branch, hq, d;
};

// Branch-local backward: the branch-key share of dQ (to workspace), dKb, dVb.
struct BwdBranchArgs {
  const void *qb, *kb, *vb, *doutb;
  const float *lseb, *ndelta_b;  // ndelta_b: -Delta of the branch rows
  float *dq_local;  // [NB, hq, d] fp32
  void *dkb, *dvb;
  const BTile *btiles;
  const int32_t *branch_off, *b_anchor;
  int32_t hq, hkv, G, d, bidir;
  float scale, scale_log2;
};

// Ring replay for dQ (query-stationary).
struct BwdDqArgs {
  const void *q, *qb, *k, *v, *dout, *doutb;
  // fp8 plans: the E4M3 q, qb, k for the scores (q/qb/k above are then their
  // exact bf16 copies, used for the K^T dS^T product); NULL otherwise
  const void *q8, *qb8, *k8;
  const float *lse, *lseb, *ndelta;  // -Delta: main rows then branch rows
  const float *lse2;                // LSE * log2(e), main rows then branch rows
  const float *dq_local;            // branch rows: branch-key share of dQ
  void *dq, *dqb;
  const QTile *qtiles;
  const int32_t *bound_main, *bound_branch;
  int32_t n_local, n_branch, hq, hkv, G, log2G, C, r, d;
  float scale, scale_log2;
  int32_t runs;  // as in FwdRingArgs
};

// Ring replay for dK/dV (key-stationary).
struct BwdDkdvArgs {
  const void *q, *qb, *k, *v, *dout, *doutb;
  const float *lse, *lseb, *ndelta, *lse2;  // ndelta: -Delta
  void *dk, *dv;
  const KTile *ktiles;
  const int32_t *bound_main, *bound_branch;
  int32_t n_local, n_branch, hq, hkv, G, log2G, d;
  float scale, scale_log2;
};

// fp32 path: per-row / per-key loops over the same visibility rules.
struct F32Shape {
  const int32_t *bound_main, *bound_branch, *branch_seq, *row_seq;
  const int32_t *cu_local, *chunk, *seq_len, *seq_a0, *branch_off, *anchor_pos;
  int32_t n_local, n_branch, n_seqs, hq, hkv, G, C, r, d;
  float scale, scale_log2;
};

// Draft-layer projection: q, k, v of rows of hidden states, per-head RMS norm
// of q and k, RoPE at each row's position, written in the attention layouts.
struct ProjArgs {
  const void *x, *w, *q_norm, *k_norm;  // bf16; q_norm/k_norm NULL: no norm
  void *q, *k, *v;
  const int32_t *bound_main;             // main rows: position, -1 for pads
  const int32_t *branch_off, *b_anchor, *anchor_pos;
  int32_t nrows, hidden, hq, hkv;
  int32_t target;  // 0: main rows, 1: branch rows
  int32_t step;    // branch rows: -1 all rows; j >= 0 step j of every local anchor
  int32_t rope;
  float eps;
  double inv_freq[64];  // theta^(-2j/128)
};

hipError_t launch_qkv_project(const ProjArgs &a, hipStream_t s);

hipError_t launch_fwd_ring_bf16(const FwdRingArgs &a, int n_tiles, hipStream_t s);
hipError_t launch_fwd_ring_fp8(const FwdRingArgs &a, int n_tiles, hipStream_t s);
hipError_t launch_fwd_branch(const FwdBranchArgs &a, int n_tiles, int dtype, int maxb, hipStream_t s);
hipError_t launch_bwd_pre(const BwdPreArgs &a, int dtype, hipStream_t s);
// E4M3 codes -> bf16 (exact), n a multiple of 8
hipError_t launch_fp8_to_bf16(const uint8_t *in, uint16_t *out, int64_t n, hipStream_t s);
hipError_t launch_bwd_branch(const BwdBranchArgs &a, int n_tiles, int dtype, int maxb, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const BwdDqArgs &a, int n_tiles, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const BwdDkdvArgs &a, int n_tiles, hipStream_t s);

hipError_t launch_fwd_ring_f32(const FwdRingArgs &a, const F32Shape &sh, hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdDqArgs &a, const F32Shape &sh, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdDkdvArgs &a, const F32Shape &sh, hipStream_t s);

}  // namespace ba
