/*
 * branch_attn.h -- C ABI of the MI355X (gfx950) draft branch attention library.
 *
 * What it computes (pages of arXiv:2609.07108):
 *   ai.info summary, Key Contributions 1 and Methodology: draft branch
 *   attention is split into a causal main-sequence part, evaluated by packed,
 *   load-balanced zigzag ring attention (K/V circulate, queries stay), and a
 *   rank-local branch part on the rank that owns the branch's anchor; the two
 *   (O, LSE) partials are merged with the online-softmax rule, which equals the
 *   full attention.
 *   rainbus analysis, core method, Eq. 2: l = log(e^lm + e^lb),
 *   O = (e^(lm-l) Om + e^(lb-l) Ob) / (e^(lm-l) + e^(lb-l)).
 *   rainbus analysis, method steps, steps two and five: ring steps over the C
 *   ranks' K/V shards forward; the backward replays the ring and accumulates
 *   gradients locally.
 *
 * On one GPU the library computes ONE context-parallel rank's share at its
 * real shape: rank r's local zigzag rows (main rows and the branch rows of the
 * anchors it owns) against every virtual ring step's K/V shard, all resident
 * in device memory. No inter-GPU traffic happens here.
 *
 * Visible key set of a query row (the definition the kernels reproduce):
 *   real main row at position p of sequence s  -> main keys of s at 0..p;
 *   branch row j of an anchor at position pa   -> main keys of s at 0..pa, plus
 *       the anchor's branch keys j' <= j (TTT chains, causal blocks) or all of
 *       them (bidirectional blocks);
 *   pad row -> nothing (O = 0, LSE = -inf); pad keys are never visible.
 * For q-head h the kv-head is h / (hq / hkv). Scores are scale * <q, k>; LSE
 * is the natural log-sum-exp of the scores.
 *
 * Zigzag layout: every sequence is padded at its tail to a multiple of 2C and
 * cut into 2C equal chunks; rank r holds chunk r then chunk 2C-1-r, sequences
 * in batch order. "Local rows" of rank r are those chunks, back to back.
 *
 * Tensor layouts (all contiguous, row-major, element type = dtype unless
 * stated; N = n_local_rows, NB = n_branch_rows):
 *   q, o, dq, do            [N,  hq,  d]
 *   k, v, dk, dv            [C,  N,   hkv, d]  shard s = rank s's local rows
 *   qb, ob, dqb, dob        [NB, hq,  d]       branch rows of the local anchors,
 *                                              anchor after anchor (branch_off)
 *   kb, vb, dkb, dvb        [NB, hkv, d]       one branch key per branch row
 *   lse                     [N,  hq]  float32
 *   lseb                    [NB, hq]  float32
 * dk/dv hold this rank's contribution to the gradient of every shard (in a
 * real ring they travel back to their owners); dq/dk/dv of pad rows are 0.
 *
 * Ownership and threading:
 *   - The caller owns every device buffer and the stream. A plan is created
 *     on the host (ba_plan_create), uploaded once to the current device
 *     (ba_plan_upload: the only call that allocates device memory; it may be
 *     called from several threads at once), and is immutable afterwards, so
 *     concurrent use on several streams is safe.
 *   - branch_attn_fwd / branch_attn_bwd never allocate and never synchronise:
 *     they validate, then enqueue kernels on the caller's stream and return.
 *     Asynchronous device faults surface at the caller's next synchronisation.
 *   - Pointers must be device pointers, 16-byte aligned.
 * Errors: every entry point returns a ba_status; no C++ exception crosses the
 * ABI and nothing is printed. ba_last_error() gives a thread-local detail
 * string for the last failing call on that thread.
 */
#ifndef BRANCH_ATTN_H
#define BRANCH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_OK = 0,
  BA_E_INVALID = 1,     /* bad argument (sizes, order, pointers, state) */
  BA_E_UNSUPPORTED = 2, /* valid but outside what the library supports */
  BA_E_WORKSPACE = 3,   /* workspace missing or smaller than required */
  BA_E_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  BA_E_OOM = 5          /* host or device allocation failed */
} ba_status;

/* Element types. BA_FP8: q, k, qb, kb hold OCP fp8 E4M3 codes (1 byte:
 * exponent bias 7, no infinities, 0x7F/0xFF NaN); v, vb, o, ob are bf16; lse
 * fp32. The forward forms the scores by fp8 matrix-core products with fp32
 * accumulation, everything after them as for BA_BF16. Per-tensor fp8 scale
 * factors of Q and K fold into the softmax scale (s = scale * <q, k>). The
 * backward takes the E4M3 values of q, k, qb, kb as bf16 (each E4M3 value is
 * a bf16 value; the copies live in the backward workspace) and runs the bf16
 * backward, except that the ring dQ kernel forms its scores by fp8 products
 * of the E4M3 codes (the same products as the forward, summed in another
 * order): dq, dk, dqb, dkb are bf16 gradients with respect to those
 * values. */
typedef enum { BA_BF16 = 0, BA_FP32 = 1, BA_FP8 = 2 } ba_dtype;

typedef enum {
  BA_BRANCH_NONE = 0,         /* main rows only: plain causal zigzag ring attention */
  BA_BRANCH_TTT = 1,          /* EAGLE-3 training-time test: every real position anchors
                                 depth_or_block chained rows; row j sees branch keys 0..j
                                 (paperlens walkthrough, "The two walls") */
  BA_BRANCH_BLOCK_BIDIR = 2,  /* DFlash: a block branch, bidirectional inside the block */
  BA_BRANCH_BLOCK_CAUSAL = 3  /* DSpark: a block branch, causal inside the block (rainbus
                                 analysis, background on the three draft families) */
} ba_branch_kind;

typedef struct ba_plan ba_plan; /* opaque, library-owned */

/* Sizes and work counts of a plan (all counts per rank). */
typedef struct {
  int32_t n_seqs, cp_degree, cp_rank, kind, hq, hkv, d, dtype;
  int32_t max_branch_len;
  int32_t run_walk;        /* 1: the forward and dQ kernels walk per-tile run lists
                              (chosen when every chunk is <= 8192 rows, or forced by
                              ba_plan_set_walk); 0: they walk the (step, chunk) segments */
  int64_t n_local_rows;    /* N: rank-local main rows, pads included */
  int64_t n_pad_rows;      /* pad rows among them */
  int64_t n_local_anchors; /* anchors owned by this rank */
  int64_t n_branch_rows;   /* NB */
  int64_t pairs_main;      /* unmasked (row, key) pairs per q-head: main rows */
  int64_t pairs_prefix;    /* branch rows x main prefix keys */
  int64_t pairs_local;     /* branch rows x own branch keys */
  int64_t pairs_total;
  size_t ws_fwd_bytes;     /* device workspace branch_attn_fwd needs */
  size_t ws_bwd_bytes;     /* device workspace branch_attn_bwd needs */
} ba_plan_info;

/* Host index arrays of a plan (library-owned, valid until ba_plan_destroy). */
typedef struct {
  const int32_t *cu_real;    /* [n_seqs+1] prefix sums of real lengths */
  const int32_t *cu_pad;     /* [n_seqs+1] prefix sums of padded lengths */
  const int32_t *cu_local;   /* [n_seqs+1] prefix sums of local rows (2 chunks each) */
  const int32_t *perm;       /* [N] local row -> global padded position cu_pad[s]+pos */
  const int32_t *is_pad;     /* [N] 1 for pad rows */
  const int32_t *pos;        /* [N] position inside its sequence */
  const int32_t *seq;        /* [N] sequence id */
  const int32_t *anchor_row; /* [A] local main row of each local anchor */
  const int32_t *anchor_pos; /* [A] its position inside the sequence */
  const int32_t *anchor_seq; /* [A] its sequence */
  const int32_t *branch_off; /* [A+1] first branch row of each local anchor */
} ba_indices;

/*
 * Build the plan of rank cp_rank of cp_degree (host only, no device calls).
 *   seqlens[n_seqs]   real lengths, in packed order, each >= 1.
 *   kind              see ba_branch_kind.
 *   depth_or_block    TTT: chain depth (rows per anchor, >= 1); block kinds:
 *                     uniform block length when branch_lens is NULL.
 *   anchors[n_anchors] block kinds only: global indices into the packed stream
 *                     of real tokens, strictly increasing (NULL/0 otherwise).
 *   branch_lens       block kinds: per-anchor block length (NULL = uniform).
 *   hq, hkv, d, dtype head configuration the plan's work lists are built for.
 * Supported: hq % hkv == 0 with hq/hkv a power of two <= 64; bf16 and fp8 need
 * d == 128, fp32 takes d == 64 or 128; branch lengths 1..64.
 * Returns BA_E_INVALID / BA_E_UNSUPPORTED with *out untouched on error.
 * Partition rule: rainbus analysis, background on context parallelism (head
 * and tail chunk per rank) and method steps, step two (N/C tokens per rank).
 */
ba_status ba_plan_create(const int32_t *seqlens, int32_t n_seqs, int32_t cp_degree,
                         int32_t cp_rank, ba_branch_kind kind, int32_t depth_or_block,
                         const int32_t *anchors, int32_t n_anchors,
                         const int32_t *branch_lens, int32_t hq, int32_t hkv, int32_t d,
                         ba_dtype dtype, ba_plan **out);

/* Copy the plan's index arrays and work lists to the CURRENT HIP device
 * (hipMalloc + synchronous copies). Must precede fwd/bwd; calling it again on
 * the same device is a no-op, on another device BA_E_INVALID. */
ba_status ba_plan_upload(ba_plan *plan);

ba_status ba_plan_get_info(const ba_plan *plan, ba_plan_info *out);

/* How the forward and dQ kernels walk each query tile's keys: mode 0 chooses
 * by chunk size (a run list built per tile when every chunk is <= 8192 rows,
 * the (step, chunk) segments otherwise), 1 forces the segments, 2 the run
 * list. Both walks visit the same keys; results agree to summation order.
 * For tests and measurement; takes effect at the next fwd/bwd call. Not
 * thread-safe against concurrent fwd/bwd calls on the same plan. */
ba_status ba_plan_set_walk(ba_plan *plan, int32_t mode);
ba_status ba_plan_get_indices(const ba_plan *plan, ba_indices *out);
void ba_plan_destroy(ba_plan *plan); /* frees host and device memory; NULL is a no-op */

/*
 * Inspection of the kernels' work lists (host copies, library-owned, valid
 * until ba_plan_destroy). which = 0: query tiles of the forward and dQ
 * kernels, 8 int32 each {kv_head, source (0 main rows, 1 branch rows), first
 * row, rows, first local row of the sequence, chunk size, smallest causal
 * bound, largest causal bound}; which = 1: key tiles of the dK/dV kernel, 12
 * int32 each {kv_head, shard, first key row in the shard, the position the
 * kernel's mask gives key 0, keys, first/end main row, first/end branch row,
 * sequence, run, run offset}: with run = 0 the keys are consecutive rows of
 * the shard; with run > 0 key k is row first + (offset + k) % run of shard
 * shard + (offset + k) / run (the chunk pairs of consecutive shards, packed
 * back to back); which = 2:
 * branch tiles, 4 int32 each {kv_head, first anchor, end anchor, rows}.
 * Tiles with zero rows/keys are padding slots. Order = launch order.
 */
ba_status ba_plan_get_worklist(const ba_plan *plan, int32_t which, const int32_t **data,
                               int64_t *n_tiles, int32_t *ints_per_tile);

typedef struct {
  float scale;                 /* softmax scale; <= 0 means 1/sqrt(d) */
  const void *q, *k, *v;       /* inputs, layouts above */
  const void *qb, *kb, *vb;    /* branch inputs; may be NULL when NB == 0 */
  void *o;                     /* [N, hq, d] */
  float *lse;                  /* [N, hq] */
  void *ob;                    /* [NB, hq, d]; NULL when NB == 0 */
  float *lseb;                 /* [NB, hq];    NULL when NB == 0 */
  void *workspace;             /* device scratch of >= ws_fwd_bytes (may be NULL if 0) */
  size_t workspace_bytes;
} ba_fwd_args;

typedef struct {
  float scale;                 /* same scale as the forward */
  const void *q, *k, *v, *qb, *kb, *vb;
  const void *o, *ob;          /* forward outputs */
  const float *lse, *lseb;     /* forward LSEs (the merged ones) */
  const void *dout, *doutb;    /* incoming gradients of o and ob */
  void *dq, *dk, *dv;          /* [N,hq,d], [C,N,hkv,d], [C,N,hkv,d]; fully overwritten */
  void *dqb, *dkb, *dvb;       /* [NB,hq,d], [NB,hkv,d], [NB,hkv,d]; fully overwritten */
  void *workspace;             /* device scratch of >= ws_bwd_bytes */
  size_t workspace_bytes;
} ba_bwd_args;

/*
 * Forward: main-sequence partial over every ring step i = 0..C-1 (shard
 * (r - i) mod C, merged in registers between steps), the rank-local branch
 * partial, and the Eq. 2 merge of the two for every branch row.
 * stream: a hipStream_t (NULL = default stream). Enqueue only.
 */
ba_status branch_attn_fwd(const ba_plan *plan, const ba_fwd_args *args, void *stream);

/*
 * The forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels and results as branch_attn_fwd,
 * with the workspace taken from a static device array of the library
 * (256 MiB, one copy per GPU, held until the process ends; its address is
 * looked up once per device by ba_plan_upload). It allocates nothing and
 * synchronises nothing.
 *   args->workspace must be NULL and args->workspace_bytes 0 (BA_E_INVALID
 *   otherwise); every other field as for branch_attn_fwd.
 *   Plans whose ws_fwd_bytes exceeds 256 MiB are rejected with BA_E_WORKSPACE
 *   before any argument is read or any kernel is enqueued.
 *   The array needs no clearing: every byte a call reads was written earlier
 *   in the same call.
 *   All calls on one GPU share the array: calls whose kernels can overlap
 *   (different streams without ordering between them) race on it and give
 *   undefined results. Calls on one stream, or ordered by events, are safe.
 */
ba_status branch_attn_fwd_static(const ba_plan *plan, const ba_fwd_args *args, void *stream);

/*
 * Backward, recomputed from the merged LSE: Delta = rowsum(dO * O), then the
 * ring replay (dQ for every local row; dK/dV for every shard), the branch-local
 * backward, and the final sums. Enqueue only.
 * Precision (bf16): as in bf16 matrix-core attention, O (in Delta), P (in the
 * forward's P V) and dS are rounded to bf16. Each rounding leaves the row sum
 * of dS slightly off its exact value 0, and dQ = scale * sum_k dS_k k_k picks
 * up that residue times whatever component the keys of a row share. For
 * keys whose shared component is up to a few times their spread the results
 * stay within bf16 attention's usual error; far beyond that (scores of a row
 * all shifted by hundreds of units together) dQ degrades in proportion to
 * the shared component. dK and dV are not affected.
 */
ba_status branch_attn_bwd(const ba_plan *plan, const ba_bwd_args *args, void *stream);

/*
 * Draft-layer projection: the step of the draft forward that produces the
 * attention inputs (rainbus analysis, method steps, step four: EAGLE-3's
 * training-time-test passes, DFlash's whole block; paperlens walkthrough,
 * "The two walls"). For rows of draft hidden states x:
 *   y = x W^T, split into hq q heads, hkv k heads, hkv v heads of d = 128;
 *   q and k per head: y / sqrt(mean(y^2) + norm_eps) * norm weight (when
 *     q_norm/k_norm are given);
 *   q and k: rotary embedding at the row's position p, rotate-half form:
 *     (y_j, y_{j+64}) turns by p * rope_theta^(-2j/128), j < 64 (when
 *     rope_theta > 0).
 * Positions: a main row sits at its position in its sequence; branch row j
 * of the anchor at position p at p + 1 + j (the token it stands for). Pad
 * main rows are written as zeros.
 * Layouts (bf16, contiguous):
 *   target 0, main rows: x [N, hidden] in local row order -> q [N, hq, d];
 *     k, v [N, hkv, d] (this rank's own shard of the k/v arrays).
 *   target 1, step -1, branch rows: x [NB, hidden] in branch-row order ->
 *     qb [NB, hq, d], kb, vb [NB, hkv, d].
 *   target 1, step j (TTT plans, 0 <= j < depth): x [A, hidden], one row per
 *     local anchor in anchor order (the step-major input of one TTT pass) ->
 *     branch row j of every anchor in qb, kb, vb; other rows are untouched.
 *   w [(hq + 2 hkv) d, hidden]: q heads, then k heads, then v heads.
 *   q_norm, k_norm [d], both or neither.
 * Needs a bf16 plan with d == 128 (BA_E_UNSUPPORTED otherwise), hidden a
 * positive multiple of 64 (BA_E_INVALID otherwise) and below 2^23
 * (BA_E_UNSUPPORTED). Rows of the output tensors not listed above are not
 * touched. Enqueue only; allocates nothing.
 */
typedef struct {
  int32_t target;     /* 0: main rows, 1: branch rows */
  int32_t step;       /* -1, or a TTT step (target 1) */
  int32_t hidden;
  float rope_theta;   /* <= 0: no rotary embedding */
  float norm_eps;
  const void *x, *w, *q_norm, *k_norm;
  void *q, *k, *v;
} ba_proj_args;

ba_status ba_qkv_project(const ba_plan *plan, const ba_proj_args *args, void *stream);

const char *ba_status_str(ba_status s);
const char *ba_last_error(void);

/*
 * Kernel timing (measurement aid; off by default). While enabled, every kernel
 * launch of fwd/bwd is bracketed by HIP events recorded on the launch stream.
 * ba_profile_read synchronises those events and returns, per kernel name, the
 * number of launches and their summed duration in milliseconds, then resets.
 * Event creation happens in ba_profile_enable, never inside fwd/bwd.
 */
typedef struct {
  char name[32];
  int64_t launches;
  double total_ms;
} ba_kernel_time;

ba_status ba_profile_enable(int32_t on, int32_t max_launches);
ba_status ba_profile_read(ba_kernel_time *out, int32_t max_entries, int32_t *n_entries);

/*
 * Matrix-core rate probe (measurement aid, not part of the attention path;
 * for callers that compare kernel rates with what the part sustains). Every
 * wave of a grid of 2048 x 256 threads runs eight independent accumulation
 * chains of bf16 32x32x16 MFMAs on register operands for `iters` iterations:
 * all-zero operands (random_operands = 0) or fixed pseudo-random bf16 values
 * in [-1, 1) that change from one MFMA to the next (random_operands != 0).
 *   sink     device buffer of at least 8192 floats (per-wave sums, written so
 *            the work is kept); sink_len its length in floats.
 *   stream   enqueued on this stream; the call then synchronises on it (unlike
 *            fwd/bwd) and creates and destroys two HIP events.
 *   *tflops  dense bf16 TFLOP/s measured with HIP events around the launch.
 * Returns BA_E_INVALID for a NULL sink/tflops, iters outside 1..2^24 or a
 * short sink, BA_E_HIP if a HIP call fails.
 */
ba_status ba_probe_mfma(int32_t random_operands, int32_t iters, float *sink, int64_t sink_len,
                        void *stream, double *tflops);

#ifdef __cplusplus
}
#endif

#endif /* BRANCH_ATTN_H */
