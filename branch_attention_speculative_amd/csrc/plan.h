// Internal plan representation shared by the host planner and the launchers.
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/branch_attn.h"

namespace ba {

// Tiling constants of the bf16 MFMA kernels (D = 128).
constexpr int kQTileVecs = 256;   // query vectors (row, head) per forward / dQ tile
constexpr int kKTileKeys = 128;   // keys per dK/dV tile
// joined chunk pairs shorter than this are packed across shards into full
// dK/dV tiles (dspark: dK/dV 12% faster; with runs of 1024-3072 keys, as in
// ttt32k, packing saved 1% of the tiles and measured 1% slower)
constexpr int kPackRunMaxKeys = 1024;
constexpr int kKBlockVecs = 64;   // query vectors per dK/dV inner block
constexpr int kMaxBranch = 64;    // longest branch the branch-local kernels accept
constexpr int kNumXcd = 8;        // MI355X: 8 accelerator complex dies, WGs dispatched round-robin
// The forward and dQ kernels walk a tile's keys through a run list built in
// LDS when every sequence's chunk is at most this many rows, and through the
// (step, chunk) segments otherwise (measured: the run list is faster on
// chunks of hundreds of rows, slightly slower on chunks of 16K rows).
constexpr int kRunWalkMaxChunk = 8192;

// Query tile of the forward / dQ kernels: consecutive rows of one source
// (main rows or branch rows) of one sequence chunk, times the G q-heads of one
// kv-head. nrows == 0 marks an empty slot.
struct QTile {
  int32_t g, src, row0, nrows;
  int32_t seq_off;  // cu_local[s]: first local row of the sequence (same in every shard)
  int32_t c;        // chunk size of the sequence
  int32_t p_min;    // smallest causal bound of its rows (-1 if a pad row is present)
  int32_t p_max;    // largest causal bound of its rows
};
static_assert(sizeof(QTile) == 32, "QTile layout");

// Key tile of the dK/dV kernel: up to kKTileKeys key rows of one sequence,
// for one kv-head, plus the local query rows that can see any of them (a
// suffix of the sequence's main rows, and of its branch rows). With run == 0
// the keys are consecutive rows krow0 .. of shard `shard`: they lie in one
// chunk, or span the shard's two chunks of the sequence when every local row
// sees both chunks or neither. With run > 0 the tile packs the joined chunk
// pairs of consecutive shards, each run = 2c rows starting at row krow0 of
// its shard: key kk is row krow0 + (run_off + kk) % run of shard
// shard + (run_off + kk) / run. Key kk is masked as if at position
// kpos0 + kk, which decides visibility exactly as the true positions do.
struct KTile {
  int32_t g, shard, krow0, kpos0;
  int32_t nkeys, qm_start, qm_end, qb_start;
  int32_t qb_end, seq, run, run_off;
};
static_assert(sizeof(KTile) == 48, "KTile layout");

// Branch-local tile: whole local anchors [a0, a1) for one kv-head.
struct BTile {
  int32_t g, a0, a1, rows;
};
static_assert(sizeof(BTile) == 16, "BTile layout");

struct DevPlan {
  int device = -1;
  void *block = nullptr;  // one allocation holding every array below
  const int32_t *bound_main = nullptr;    // [N] position, -1 for pads
  const int32_t *bound_branch = nullptr;  // [NB] anchor position
  const int32_t *b_anchor = nullptr;      // [NB] local anchor of each branch row
  const int32_t *branch_off = nullptr;    // [A+1]
  const QTile *qtiles = nullptr;
  const KTile *ktiles = nullptr;
  const BTile *btiles = nullptr;
  const int32_t *row_seq = nullptr;       // [N] sequence of each main row
  const int32_t *branch_seq = nullptr;    // [NB] sequence of each branch row
  const int32_t *cu_local = nullptr;      // [S+1]
  const int32_t *chunk = nullptr;         // [S] chunk size per sequence
  const int32_t *seq_len = nullptr;       // [S] real length per sequence
  const int32_t *seq_a0 = nullptr;        // [S+1] first local anchor of each sequence
  const int32_t *anchor_pos = nullptr;    // [A]
};

}  // namespace ba

struct ba_plan {
  // configuration
  int32_t n_seqs = 0, C = 0, r = 0, kind = 0, depth_or_block = 0;
  int32_t hq = 0, hkv = 0, d = 0, dtype = 0, G = 0, max_branch_len = 0;
  // per sequence
  std::vector<int32_t> L, P, c, cu_real, cu_pad, cu_local;
  // per local main row
  std::vector<int32_t> pos, seq, perm, is_pad, bound_main;
  // per local anchor
  std::vector<int32_t> anchor_row, anchor_pos, anchor_seq, branch_off, seq_a0;
  // per branch row
  std::vector<int32_t> b_anchor, bound_branch, branch_seq;
  // work lists
  std::vector<ba::QTile> qtiles;
  std::vector<ba::KTile> ktiles;
  std::vector<ba::BTile> btiles;
  int64_t n_local = 0, n_branch = 0, n_pad = 0;
  int64_t pairs_main = 0, pairs_prefix = 0, pairs_local = 0;
  size_t ws_fwd = 0, ws_bwd = 0;
  int32_t run_walk_auto = 0;  // every chunk <= kRunWalkMaxChunk
  int32_t walk_mode = 0;      // 0: automatic, 1: segments, 2: run list (ba_plan_set_walk)
  ba::DevPlan dev;
  // guards dev: ba_plan_upload may run on several threads at once, and
  // fwd/bwd read dev under it
  mutable std::mutex dev_mu;
};

namespace ba {
// Whether the forward and dQ kernels walk run lists for this plan.
inline bool uses_run_walk(const ba_plan &p) {
  return p.walk_mode == 2 || (p.walk_mode == 0 && p.run_walk_auto != 0);
}
// Thread-local error detail used by every entry point.
void set_error(const std::string &msg);
const char *get_error();
ba_status fail(ba_status st, const std::string &msg);
// Workspace layout.
size_t ws_fwd_bytes(const ba_plan &p);
size_t ws_bwd_bytes(const ba_plan &p);
}  // namespace ba
