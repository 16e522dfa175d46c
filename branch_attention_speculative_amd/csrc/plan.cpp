// Host-side planner: packed zigzag split, anchor -> branch index, pair
// counts, and the work lists of the kernels. No device calls in this file.
//
// Partition rule (rainbus analysis of arXiv:2609.07108, background section on
// context parallelism, and method steps, step two): every sequence is padded
// at its tail to a multiple of 2C and cut into 2C equal chunks; rank r holds
// chunk r (head) and chunk 2C-1-r (tail), so each rank holds N/C tokens and
// the causal work is balanced. Branches live on the rank that owns their
// anchor (ai.info summary, Key Contributions 1).

#include <algorithm>
#include <cmath>
#include <limits>
#include <memory>
#include <new>
#include <numeric>
#include <string>
#include <vector>

#include "plan.h"

namespace ba {

static thread_local std::string g_err;

void set_error(const std::string &msg) { g_err = msg; }
const char *get_error() { return g_err.c_str(); }
ba_status fail(ba_status st, const std::string &msg) {
  g_err = msg;
  return st;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Forward workspace: the main-sequence partial (O_m normalised, fp32, and its
// LSE) of every branch row, handed from the ring kernel to the Eq. 2 merge.
size_t ws_fwd_bytes(const ba_plan &p) {
  if (p.n_branch == 0) return 0;
  return align256(size_t(p.n_branch) * p.hq * p.d * 4) + align256(size_t(p.n_branch) * p.hq * 4);
}

// Backward workspace: Delta and LSE * log2(e) of every row (main then
// branch, fp32) and the branch-local share of dQ of every branch row (fp32).
// fp8 plans add bf16 copies of q, k, qb and kb, in that order (every E4M3
// value is a bf16 value, so the backward runs on those copies).
size_t ws_bwd_bytes(const ba_plan &p) {
  size_t b = 2 * align256(size_t(p.n_local + p.n_branch) * p.hq * 4) +
             align256(size_t(p.n_branch) * p.hq * p.d * 4);
  if (p.dtype == BA_FP8)
    b += align256(size_t(p.n_local) * p.hq * p.d * 2) +
         align256(size_t(p.C) * p.n_local * p.hkv * p.d * 2) +
         align256(size_t(p.n_branch) * p.hq * p.d * 2) + align256(size_t(p.n_branch) * p.hkv * p.d * 2);
  return b;
}

// Order tiles for an XCD-round-robin dispatch: tiles arrive in locality order
// (same kv-head and sequence together); the list is cut into kNumXcd
// contiguous parts of about equal cost, each part is sorted heaviest first,
// and the parts are interleaved so that workgroup b runs on XCD b % kNumXcd
// and meets its part in order. Empty slots pad unequal parts.
template <class T>
static std::vector<T> xcd_order(const std::vector<T> &tiles, const std::vector<double> &cost,
                                const T &empty) {
  const size_t n = tiles.size();
  std::vector<std::vector<size_t>> part(kNumXcd);
  double total = 0;
  for (double c : cost) total += c;
  double acc = 0;
  int x = 0;
  for (size_t i = 0; i < n; ++i) {
    part[x].push_back(i);
    acc += cost[i];
    if (x < kNumXcd - 1 && acc >= total * (x + 1) / kNumXcd) ++x;
  }
  size_t longest = 0;
  for (auto &pt : part) {
    std::stable_sort(pt.begin(), pt.end(), [&](size_t a, size_t b) { return cost[a] > cost[b]; });
    longest = std::max(longest, pt.size());
  }
  std::vector<T> out(longest * kNumXcd, empty);
  for (int xx = 0; xx < kNumXcd; ++xx)
    for (size_t i = 0; i < part[xx].size(); ++i) out[i * kNumXcd + xx] = tiles[part[xx][i]];
  return out;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

static ba_status build(ba_plan &p, const int32_t *seqlens, const int32_t *anchors,
                       int32_t n_anchors, const int32_t *branch_lens) {
  const int S = p.n_seqs, C = p.C, r = p.r;
  const int64_t two_c = 2 * int64_t(C);
  p.L.resize(S);
  p.P.resize(S);
  p.c.resize(S);
  p.cu_real.assign(S + 1, 0);
  p.cu_pad.assign(S + 1, 0);
  p.cu_local.assign(S + 1, 0);
  int64_t real = 0, padded = 0, local = 0;
  for (int s = 0; s < S; ++s) {
    if (seqlens[s] < 1) return fail(BA_E_INVALID, "seqlens[" + std::to_string(s) + "] < 1");
    const int64_t L = seqlens[s];
    const int64_t P = (L + two_c - 1) / two_c * two_c;
    real += L;
    padded += P;
    local += P / C;
    if (padded > std::numeric_limits<int32_t>::max() / 2)
      return fail(BA_E_UNSUPPORTED, "packed padded length exceeds 2^30 tokens");
    p.L[s] = int32_t(L);
    p.P[s] = int32_t(P);
    p.c[s] = int32_t(P / two_c);
    p.cu_real[s + 1] = int32_t(real);
    p.cu_pad[s + 1] = int32_t(padded);
    p.cu_local[s + 1] = int32_t(local);
  }
  p.n_local = local;

  // local rows of rank r: head chunk r, then tail chunk 2C-1-r, per sequence
  p.pos.resize(local);
  p.seq.resize(local);
  p.perm.resize(local);
  p.is_pad.resize(local);
  p.bound_main.resize(local);
  for (int s = 0; s < S; ++s) {
    const int32_t c = p.c[s];
    int32_t row = p.cu_local[s];
    for (int half = 0; half < 2; ++half) {
      const int64_t chunk = half == 0 ? r : 2 * int64_t(C) - 1 - r;
      for (int32_t i = 0; i < c; ++i, ++row) {
        const int32_t ps = int32_t(chunk * c + i);
        p.pos[row] = ps;
        p.seq[row] = s;
        p.perm[row] = p.cu_pad[s] + ps;
        p.is_pad[row] = ps >= p.L[s] ? 1 : 0;
        p.bound_main[row] = ps >= p.L[s] ? -1 : ps;
      }
    }
  }
  p.n_pad = 0;
  for (int32_t x : p.is_pad) p.n_pad += x;

  // anchors owned by this rank, in local row order
  std::vector<int32_t> lens;
  if (p.kind == BA_BRANCH_TTT) {
    if (p.depth_or_block < 1 || p.depth_or_block > kMaxBranch)
      return fail(p.depth_or_block < 1 ? BA_E_INVALID : BA_E_UNSUPPORTED,
                  "TTT depth must be in 1.." + std::to_string(kMaxBranch));
    for (int64_t row = 0; row < local; ++row) {
      if (p.is_pad[row]) continue;
      p.anchor_row.push_back(int32_t(row));
      p.anchor_pos.push_back(p.pos[row]);
      p.anchor_seq.push_back(p.seq[row]);
      lens.push_back(p.depth_or_block);
    }
  } else if (p.kind == BA_BRANCH_BLOCK_BIDIR || p.kind == BA_BRANCH_BLOCK_CAUSAL) {
    if (n_anchors < 0) return fail(BA_E_INVALID, "n_anchors < 0");
    if (n_anchors > 0 && anchors == nullptr) return fail(BA_E_INVALID, "anchors is NULL");
    if (branch_lens == nullptr && (p.depth_or_block < 1 || p.depth_or_block > kMaxBranch))
      return fail(p.depth_or_block < 1 ? BA_E_INVALID : BA_E_UNSUPPORTED,
                  "block length must be in 1.." + std::to_string(kMaxBranch));
    struct A {
      int32_t row, pos, seq, len;
    };
    std::vector<A> mine;
    for (int32_t i = 0; i < n_anchors; ++i) {
      const int64_t a = anchors[i];
      if (a < 0 || a >= real) return fail(BA_E_INVALID, "anchor " + std::to_string(i) + " out of range");
      if (i > 0 && anchors[i] <= anchors[i - 1])
        return fail(BA_E_INVALID, "anchors must be strictly increasing");
      const int32_t len = branch_lens ? branch_lens[i] : p.depth_or_block;
      if (len < 1) return fail(BA_E_INVALID, "branch length < 1");
      if (len > kMaxBranch)
        return fail(BA_E_UNSUPPORTED, "branch length > " + std::to_string(kMaxBranch));
      const int32_t s = int32_t(std::upper_bound(p.cu_real.begin(), p.cu_real.end(), int32_t(a)) -
                                p.cu_real.begin() - 1);
      const int32_t ps = int32_t(a - p.cu_real[s]);
      const int32_t c = p.c[s];
      const int32_t chunk = ps / c;
      const int32_t owner = chunk < C ? chunk : 2 * C - 1 - chunk;
      if (owner != r) continue;
      const int32_t row = p.cu_local[s] + (chunk < C ? ps - chunk * c : c + ps - chunk * c);
      mine.push_back({row, ps, s, len});
    }
    std::stable_sort(mine.begin(), mine.end(), [](const A &x, const A &y) { return x.row < y.row; });
    for (const A &x : mine) {
      p.anchor_row.push_back(x.row);
      p.anchor_pos.push_back(x.pos);
      p.anchor_seq.push_back(x.seq);
      lens.push_back(x.len);
    }
  } else if (p.kind != BA_BRANCH_NONE) {
    return fail(BA_E_INVALID, "unknown branch kind");
  }
  const int64_t A = int64_t(p.anchor_row.size());
  p.branch_off.assign(A + 1, 0);
  int64_t nb = 0;
  p.max_branch_len = 0;
  for (int64_t a = 0; a < A; ++a) {
    nb += lens[a];
    if (nb > std::numeric_limits<int32_t>::max() / 2)
      return fail(BA_E_UNSUPPORTED, "too many branch rows");
    p.branch_off[a + 1] = int32_t(nb);
    p.max_branch_len = std::max(p.max_branch_len, lens[a]);
  }
  p.n_branch = nb;
  p.b_anchor.resize(nb);
  p.bound_branch.resize(nb);
  p.branch_seq.resize(nb);
  for (int64_t a = 0; a < A; ++a)
    for (int32_t b = p.branch_off[a]; b < p.branch_off[a + 1]; ++b) {
      p.b_anchor[b] = int32_t(a);
      p.bound_branch[b] = p.anchor_pos[a];
      p.branch_seq[b] = p.anchor_seq[a];
    }

  // unmasked pairs per q-head, straight from the visibility rules
  p.pairs_main = p.pairs_prefix = p.pairs_local = 0;
  for (int64_t row = 0; row < local; ++row)
    if (!p.is_pad[row]) p.pairs_main += int64_t(p.pos[row]) + 1;
  for (int64_t a = 0; a < A; ++a) {
    const int64_t n = lens[a];
    p.pairs_prefix += n * (int64_t(p.anchor_pos[a]) + 1);
    p.pairs_local += p.kind == BA_BRANCH_BLOCK_BIDIR ? n * n : n * (n + 1) / 2;
  }

  // ---- work lists ---------------------------------------------------------
  const int G = p.G;
  const int R = std::max(1, kQTileVecs / G);  // rows per query tile
  // first/last local anchor of every sequence chunk
  std::vector<QTile> qt;
  std::vector<double> qc;
  auto emit_rows = [&](int src, int32_t lo, int32_t hi, int s) {
    for (int32_t row0 = lo; row0 < hi; row0 += R) {
      const int32_t n = std::min<int32_t>(R, hi - row0);
      int32_t pmin = std::numeric_limits<int32_t>::max(), pmax = -1;
      for (int32_t i = row0; i < row0 + n; ++i) {
        const int32_t b = src == 0 ? p.bound_main[i] : p.bound_branch[i];
        pmin = std::min(pmin, b);
        pmax = std::max(pmax, b);
      }
      for (int g = 0; g < p.hkv; ++g) {
        qt.push_back(QTile{g, src, row0, n, p.cu_local[s], p.c[s], pmin, pmax});
        qc.push_back(double(n) * G * (double(pmax) + 2.0));
      }
    }
  };
  {
    // kv-head outermost keeps tiles that share K/V together before the XCD split
    std::vector<QTile> by_head;
    std::vector<double> by_head_cost;
    int64_t a = 0;
    for (int s = 0; s < S; ++s) {
      const int32_t c = p.c[s];
      const int32_t base = p.cu_local[s];
      for (int half = 0; half < 2; ++half) {
        const int32_t lo = base + half * c, hi = lo + c;
        emit_rows(0, lo, hi, s);
        int64_t a0 = a;
        while (a < A && p.anchor_seq[a] == s && p.anchor_row[a] < hi) ++a;
        if (a > a0) emit_rows(1, p.branch_off[a0], p.branch_off[a], s);
      }
    }
    for (int g = 0; g < p.hkv; ++g)
      for (size_t i = 0; i < qt.size(); ++i)
        if (qt[i].g == g) {
          by_head.push_back(qt[i]);
          by_head_cost.push_back(qc[i]);
        }
    p.qtiles = xcd_order(by_head, by_head_cost, QTile{0, 0, 0, 0, 0, 1, -1, -1});
  }
  {
    // key tiles: every row of every shard is covered exactly once per kv-head
    std::vector<int32_t> &seq_a0 = p.seq_a0;  // first local anchor of each sequence
    seq_a0.assign(S + 1, 0);
    {
      int64_t a = 0;
      for (int s = 0; s < S; ++s) {
        seq_a0[s] = int32_t(a);
        while (a < A && p.anchor_seq[a] == s) ++a;
      }
      seq_a0[S] = int32_t(A);
    }
    std::vector<KTile> kt;
    std::vector<double> kc;
    for (int g = 0; g < p.hkv; ++g)
      for (int s = 0; s < S; ++s) {
        const int32_t c = p.c[s];
        const int32_t base = p.cu_local[s];
        // real main rows of s form a prefix of [base, base+2c) with increasing positions
        int32_t real_end = base;
        while (real_end < base + 2 * c && !p.is_pad[real_end]) ++real_end;
        const int32_t a_lo = seq_a0[s], a_hi = seq_a0[s + 1];
        // The keys of shard sh for sequence s are its chunks sh and 2C-1-sh,
        // stored as 2c consecutive rows. When no chunk of this rank lies
        // between them (sh > r) and the later one holds no pad, every local
        // row sees either all 2c keys or none, so they are cut into tiles
        // as one run (fewer partial tiles for short chunks). A tile that
        // spans the two chunks takes kpos0 = (its largest key position) -
        // (nkeys - 1): the in-kernel test kpos0 + kk <= bound then holds for
        // every key and every row in its range, as the true positions do.
        auto emit = [&](int sh, int32_t row_off, int32_t nk, int32_t pos_first, int32_t pos_last,
                        int32_t run = 0, int32_t run_off = 0) {
          KTile t{};
          t.g = g;
          t.shard = sh;
          t.krow0 = base + row_off;
          t.nkeys = nk;
          t.kpos0 = pos_last - (nk - 1);
          t.run = run;
          t.run_off = run_off;
          // main rows with bound >= the smallest key position
          const int32_t qs = int32_t(
              std::lower_bound(p.pos.begin() + base, p.pos.begin() + real_end, pos_first) -
              p.pos.begin());
          t.qm_start = qs;
          t.qm_end = std::max(qs, real_end);
          // branch rows whose anchor position >= the smallest key position
          const int32_t as = int32_t(std::lower_bound(p.anchor_pos.begin() + a_lo,
                                                      p.anchor_pos.begin() + a_hi, pos_first) -
                                     p.anchor_pos.begin());
          t.qb_start = p.branch_off[as];
          t.qb_end = p.branch_off[a_hi];
          t.seq = s;
          kt.push_back(t);
          kc.push_back(double(t.nkeys) * G *
                           (double(t.qm_end - t.qm_start) + double(t.qb_end - t.qb_start)) +
                       1.0);
        };
        // The joined shards are sh0 .. C-1 (the condition holds from some
        // shard on). All of them are seen, in full, by the same rows (this
        // rank's tail chunk and the anchors in it), so when there are two or
        // more their runs are packed back to back into full tiles: key v of
        // the packed sequence is row v % 2c of shard sh0 + v / 2c. With short
        // chunks this removes most partial tiles, whose idle wave pairs
        // leave a SIMD without work. Runs of kPackRunMaxKeys keys or more
        // waste little in their one partial tile and stay unpacked.
        int sh0 = C;
        for (int sh = C - 1; sh > r && int64_t(2 * C - sh) * c <= p.L[s]; --sh) sh0 = sh;
        const int n_joined = 2 * c < kPackRunMaxKeys ? C - sh0 : 0;
        if (n_joined >= 2) {
          const int32_t run = 2 * c;
          auto pos_of = [&](int64_t v) {
            const int sh = sh0 + int(v / run);
            const int32_t i = int32_t(v % run);
            return i < c ? sh * c + i : (2 * C - 1 - sh) * c + (i - c);
          };
          const int64_t total = int64_t(n_joined) * run;
          for (int64_t v0 = 0; v0 < total; v0 += kKTileKeys) {
            const int32_t nk = int32_t(std::min<int64_t>(kKTileKeys, total - v0));
            int32_t pmin = INT32_MAX, pmax = INT32_MIN;
            for (int64_t v = v0; v < v0 + nk; ++v) {
              pmin = std::min(pmin, pos_of(v));
              pmax = std::max(pmax, pos_of(v));
            }
            emit(sh0 + int(v0 / run), 0, nk, pmin, pmax, run, int32_t(v0 % run));
          }
        }
        for (int sh = 0; sh < C; ++sh) {
          const int32_t tail = 2 * C - 1 - sh;
          const bool joined = sh > r && int64_t(tail + 1) * c <= p.L[s];
          if (joined && n_joined >= 2) continue;  // packed above
          if (joined) {
            // row i of the run: chunk sh for i < c, chunk tail after
            auto pos_of = [&](int32_t i) { return i < c ? sh * c + i : tail * c + (i - c); };
            for (int32_t off = 0; off < 2 * c; off += kKTileKeys) {
              const int32_t nk = std::min<int32_t>(kKTileKeys, 2 * c - off);
              emit(sh, off, nk, pos_of(off), pos_of(off + nk - 1));
            }
          } else {
            for (int half = 0; half < 2; ++half) {
              const int32_t chunk = half == 0 ? sh : tail;
              for (int32_t off = 0; off < c; off += kKTileKeys) {
                const int32_t nk = std::min<int32_t>(kKTileKeys, c - off);
                emit(sh, half * c + off, nk, chunk * c + off, chunk * c + off + nk - 1);
              }
            }
          }
        }
      }
    KTile empty{};
    p.ktiles = xcd_order(kt, kc, empty);
  }
  {
    std::vector<BTile> bt;
    std::vector<double> bc;
    // whole anchors, at most kMaxBranch rows (the LDS staging size) and at
    // most 128 query vectors per tile unless a single anchor needs more
    const int64_t cap = 128;
    for (int g = 0; g < p.hkv; ++g) {
      int64_t a = 0;
      while (a < A) {
        const int64_t a0 = a;
        int64_t rows = 0;
        while (a < A) {
          const int64_t len = p.branch_off[a + 1] - p.branch_off[a];
          if (rows > 0 && (rows + len > kMaxBranch || (rows + len) * G > cap)) break;
          rows += len;
          ++a;
        }
        bt.push_back(BTile{g, int32_t(a0), int32_t(a), int32_t(rows)});
        bc.push_back(double(rows) * G * p.max_branch_len + 1.0);
      }
    }
    p.btiles = xcd_order(bt, bc, BTile{0, 0, 0, 0});
  }
  p.ws_fwd = ws_fwd_bytes(p);
  p.ws_bwd = ws_bwd_bytes(p);
  p.run_walk_auto = 1;
  for (int32_t c : p.c)
    if (c > kRunWalkMaxChunk) p.run_walk_auto = 0;
  return BA_OK;
}

}  // namespace ba

using ba::fail;

extern "C" ba_status ba_plan_create(const int32_t *seqlens, int32_t n_seqs, int32_t cp_degree,
                                    int32_t cp_rank, ba_branch_kind kind, int32_t depth_or_block,
                                    const int32_t *anchors, int32_t n_anchors,
                                    const int32_t *branch_lens, int32_t hq, int32_t hkv, int32_t d,
                                    ba_dtype dtype, ba_plan **out) {
  try {
    if (out == nullptr) return fail(BA_E_INVALID, "out is NULL");
    if (seqlens == nullptr || n_seqs < 1) return fail(BA_E_INVALID, "need at least one sequence");
    if (cp_degree < 1 || cp_degree > 64) return fail(BA_E_INVALID, "cp_degree must be in 1..64");
    if (cp_rank < 0 || cp_rank >= cp_degree) return fail(BA_E_INVALID, "cp_rank out of range");
    if (kind < BA_BRANCH_NONE || kind > BA_BRANCH_BLOCK_CAUSAL)
      return fail(BA_E_INVALID, "unknown branch kind");
    if (hq < 1 || hkv < 1 || hq % hkv != 0) return fail(BA_E_INVALID, "need hq % hkv == 0");
    const int G = hq / hkv;
    if (!ba::pow2(G) || G > 64) return fail(BA_E_UNSUPPORTED, "hq/hkv must be a power of two <= 64");
    if (dtype == BA_BF16) {
      if (d != 128) return fail(BA_E_UNSUPPORTED, "bf16 path supports d == 128");
    } else if (dtype == BA_FP32) {
      if (d != 64 && d != 128) return fail(BA_E_UNSUPPORTED, "fp32 path supports d == 64 or 128");
    } else if (dtype == BA_FP8) {
      if (d != 128) return fail(BA_E_UNSUPPORTED, "fp8 path supports d == 128");
    } else {
      return fail(BA_E_INVALID, "unknown dtype");
    }
    if ((kind == BA_BRANCH_NONE || kind == BA_BRANCH_TTT) && n_anchors != 0)
      return fail(BA_E_INVALID, "anchors are only taken by the block kinds");
    auto p = std::unique_ptr<ba_plan>(new ba_plan());
    p->n_seqs = n_seqs;
    p->C = cp_degree;
    p->r = cp_rank;
    p->kind = kind;
    p->depth_or_block = depth_or_block;
    p->hq = hq;
    p->hkv = hkv;
    p->d = d;
    p->dtype = dtype;
    p->G = G;
    const ba_status st = ba::build(*p, seqlens, anchors, n_anchors, branch_lens);
    if (st != BA_OK) return st;
    *out = p.release();
    return BA_OK;
  } catch (const std::bad_alloc &) {
    return fail(BA_E_OOM, "host allocation failed while planning");
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error while planning");
  }
}

extern "C" ba_status ba_plan_set_walk(ba_plan *p, int32_t mode) {
  if (p == nullptr) return fail(BA_E_INVALID, "plan is NULL");
  if (mode < 0 || mode > 2) return fail(BA_E_INVALID, "walk mode must be 0, 1 or 2");
  p->walk_mode = mode;
  return BA_OK;
}

extern "C" ba_status ba_plan_get_info(const ba_plan *p, ba_plan_info *out) {
  if (p == nullptr || out == nullptr) return fail(BA_E_INVALID, "NULL argument");
  ba_plan_info i{};
  i.n_seqs = p->n_seqs;
  i.cp_degree = p->C;
  i.cp_rank = p->r;
  i.kind = p->kind;
  i.hq = p->hq;
  i.hkv = p->hkv;
  i.d = p->d;
  i.dtype = p->dtype;
  i.max_branch_len = p->max_branch_len;
  i.run_walk = ba::uses_run_walk(*p) ? 1 : 0;
  i.n_local_rows = p->n_local;
  i.n_pad_rows = p->n_pad;
  i.n_local_anchors = int64_t(p->anchor_row.size());
  i.n_branch_rows = p->n_branch;
  i.pairs_main = p->pairs_main;
  i.pairs_prefix = p->pairs_prefix;
  i.pairs_local = p->pairs_local;
  i.pairs_total = p->pairs_main + p->pairs_prefix + p->pairs_local;
  i.ws_fwd_bytes = p->ws_fwd;
  i.ws_bwd_bytes = p->ws_bwd;
  *out = i;
  return BA_OK;
}

extern "C" ba_status ba_plan_get_indices(const ba_plan *p, ba_indices *out) {
  if (p == nullptr || out == nullptr) return fail(BA_E_INVALID, "NULL argument");
  out->cu_real = p->cu_real.data();
  out->cu_pad = p->cu_pad.data();
  out->cu_local = p->cu_local.data();
  out->perm = p->perm.data();
  out->is_pad = p->is_pad.data();
  out->pos = p->pos.data();
  out->seq = p->seq.data();
  out->anchor_row = p->anchor_row.data();
  out->anchor_pos = p->anchor_pos.data();
  out->anchor_seq = p->anchor_seq.data();
  out->branch_off = p->branch_off.data();
  return BA_OK;
}

extern "C" ba_status ba_plan_get_worklist(const ba_plan *p, int32_t which, const int32_t **data,
                                          int64_t *n_tiles, int32_t *ints_per_tile) {
  if (p == nullptr || data == nullptr || n_tiles == nullptr || ints_per_tile == nullptr)
    return fail(BA_E_INVALID, "NULL argument");
  switch (which) {
    case 0:
      *data = reinterpret_cast<const int32_t *>(p->qtiles.data());
      *n_tiles = int64_t(p->qtiles.size());
      *ints_per_tile = int32_t(sizeof(ba::QTile) / 4);
      return BA_OK;
    case 1:
      *data = reinterpret_cast<const int32_t *>(p->ktiles.data());
      *n_tiles = int64_t(p->ktiles.size());
      *ints_per_tile = int32_t(sizeof(ba::KTile) / 4);
      return BA_OK;
    case 2:
      *data = reinterpret_cast<const int32_t *>(p->btiles.data());
      *n_tiles = int64_t(p->btiles.size());
      *ints_per_tile = int32_t(sizeof(ba::BTile) / 4);
      return BA_OK;
  }
  return fail(BA_E_INVALID, "which must be 0, 1 or 2");
}

extern "C" const char *ba_status_str(ba_status s) {
  switch (s) {
    case BA_OK: return "BA_OK";
    case BA_E_INVALID: return "BA_E_INVALID";
    case BA_E_UNSUPPORTED: return "BA_E_UNSUPPORTED";
    case BA_E_WORKSPACE: return "BA_E_WORKSPACE";
    case BA_E_HIP: return "BA_E_HIP";
    case BA_E_OOM: return "BA_E_OOM";
  }
  return "BA_E_UNKNOWN";
}

extern "C" const char *ba_last_error(void) { return ba::get_error(); }
