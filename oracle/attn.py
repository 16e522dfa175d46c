"""Oracle: dense masked branch attention, its backward, and the split form
(test infrastructure only).

Definitions followed (pages of arXiv:2609.07108):

* ai.info summary, Methodology: every branch query looks at the causal prefix
  of the main sequence and at a small set of keys of its own branch; the main
  part is ordinary causal attention; combining the two parts with the
  log-sum-exp rule equals computing the full attention at once.
* paperlens walkthrough, "The two walls": EAGLE-3 training-time test grows a
  branch from every position; DFlash emits a block in one pass.
* rainbus analysis, background section on the three draft families: DSpark
  restores left-to-right causality inside the block (read here as a causal
  intra-block mask, as the DSpark-style workload states).
* rainbus analysis, core method, Eq. 2: l = log(e^lm + e^lb) and
  O = (e^(lm-l) Om + e^(lb-l) Ob) / (e^(lm-l) + e^(lb-l)).
* rainbus analysis, method steps, steps two and five: K/V circulate around the
  ring while queries stay; the backward replays the ring and accumulates
  gradients locally.

Visible key set V(q) of a query row (the plain definition this module writes
out, with the readings taken where the pages are silent):

* real main row at position p of sequence s: main keys of s at 0..p;
* branch row j of an anchor at position pa (branch length n): main keys of s
  at 0..pa, plus that anchor's branch keys j' <= j (TTT chains, causal blocks)
  or all j' < n (bidirectional blocks);
* pad row: nothing, so O = 0 and LSE = -inf; pad keys are in no V(q).

For q-head h, kv-head g = h // (Hq/Hkv): s_k = scale <Q[q,h], K[k,g]>,
LSE_q = ln sum_{k in V(q)} e^{s_k}, O = sum_k e^{s_k - LSE_q} V[k,g].
Backward: P = e^{s - LSE}, Delta = <dO, O>, dV = P^T dO, dP = dO V^T,
dS = P (dP - Delta), dQ = scale dS K, dK = scale dS^T Q, with dK/dV summed over
the q-heads of a kv group. dK/dV of the main keys are this rank's partial
contribution for every shard.

Tensor layouts (the library's, so inputs can be shared): q [N_loc, Hq, D];
k, v [C, N_loc, Hkv, D] (shard s in rank s's local row order); qb [N_b, Hq, D];
kb, vb [N_b, Hkv, D]; lse [rows, Hq] natural log.

Parity: pinned (tests/test_oracle_attn.py: pure-Python brute force on the
unpermuted batch, torch SDPA reduction, K = 0 closed form, one-hot V, finite
differences, fp32 vs fp64 bound, gradient sum rules, split = unsplit). The
row-sampled form ``attn_rows`` (o, lse, dq and its dK/dV accumulation) and the
subset form ``attn_subset`` (every output) are pinned against the dense
``attn_fwd``/``attn_bwd`` on every row of small cases.
"""

import numpy as np

from . import pack as _pack


def _scale(D, scale):
    return 1.0 / np.sqrt(D) if (scale is None or scale <= 0) else float(scale)


def _seq_main_key_index(layout, s):
    """(shard, local row) of each REAL position 0..L_s-1 of sequence ``s``,
    found by scanning every shard's own local row order."""
    C, L = layout["C"], layout["L"]
    shard_of = np.full(int(L[s]), -1, dtype=np.int64)
    row_of = np.full(int(L[s]), -1, dtype=np.int64)
    for sh in range(C):
        seq, pos = _pack.shard_positions(layout, sh)
        rows = np.nonzero((seq == s) & (pos < L[s]))[0]
        shard_of[pos[rows]] = sh
        row_of[pos[rows]] = rows
    assert np.all(shard_of >= 0), "every real position must live on exactly one shard"
    return shard_of, row_of


def _seq_problem(layout, br, s):
    """Query rows, key list and visibility mask for sequence ``s``.

    Returns (q_main_rows, q_branch_rows, key_shard, key_row, key_branch_rows,
    mask) where the key list is [real main positions 0..L_s-1 in order] then
    [branch keys of the local anchors of s], and mask[i, t] says whether query
    i (main rows first, then branch rows) sees key t."""
    L = int(layout["L"][s])
    kind = br["kind"]
    q_main = np.nonzero(layout["seq"] == s)[0]
    anchors = np.nonzero(br["anchor_seq"] == s)[0] if br["n_branch"] else np.zeros(0, np.int64)
    q_branch = np.nonzero(np.isin(br["b_anchor"], anchors))[0] if br["n_branch"] else np.zeros(0, np.int64)
    key_shard, key_row = _seq_main_key_index(layout, s)
    key_branch = q_branch  # branch keys are stored row-for-row with branch queries

    nq_m, nq_b, nk_m, nk_b = q_main.size, q_branch.size, L, key_branch.size
    mask = np.zeros((nq_m + nq_b, nk_m + nk_b), dtype=bool)
    key_pos = np.arange(L)
    # main rows: causal over main keys, pads see nothing
    for i, row in enumerate(q_main):
        if layout["is_pad"][row]:
            continue
        p = layout["pos"][row]
        mask[i, :nk_m] = key_pos <= p
    # branch rows: prefix up to the anchor (inclusive) plus own branch keys
    for i, brow in enumerate(q_branch):
        a = br["b_anchor"][brow]
        pa = br["anchor_pos"][a]
        mask[nq_m + i, :nk_m] = key_pos <= pa
        same = br["b_anchor"][key_branch] == a
        if kind == _pack.KIND_BLOCK_BIDIR:
            vis = same
        else:
            vis = same & (br["b_j"][key_branch] <= br["b_j"][brow])
        mask[nq_m + i, nk_m:] = vis
    return q_main, q_branch, key_shard, key_row, key_branch, mask


def _masked_softmax(S, mask):
    """Row-wise (LSE, P) of scores S under a boolean mask; fully masked rows
    give LSE = -inf and P = 0."""
    S = np.where(mask, S, -np.inf)
    m = np.max(S, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.where(mask, np.exp(S - m), 0.0)
    tot = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, tot)))
    P = np.where(empty, 0.0, e / np.where(empty, 1.0, tot))
    return lse[..., 0], P


def _gather(layout, br, s, q, k, v, qb, kb, vb, dtype):
    qm, qbr, ksh, krow, kbr, mask = _seq_problem(layout, br, s)
    Q = q[qm].astype(dtype)
    K = k[ksh, krow].astype(dtype)
    V = v[ksh, krow].astype(dtype)
    if qbr.size:
        Q = np.concatenate([Q, qb[qbr].astype(dtype)], axis=0)
        K = np.concatenate([K, kb[kbr].astype(dtype)], axis=0)
        V = np.concatenate([V, vb[kbr].astype(dtype)], axis=0)
    return qm, qbr, ksh, krow, kbr, mask, Q, K, V


def attn_fwd(layout, br, q, k, v, qb=None, kb=None, vb=None, scale=None, dtype=np.float32):
    """Dense masked forward over the full visible key set of every local row
    (main rows and branch rows). Returns (o, lse, ob, lseb) in ``dtype``."""
    N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = _scale(D, scale)
    nb = br["n_branch"]
    o = np.zeros((N, Hq, D), dtype)
    lse = np.full((N, Hq), -np.inf, dtype)
    ob = np.zeros((nb, Hq, D), dtype)
    lseb = np.full((nb, Hq), -np.inf, dtype)
    for s in range(layout["L"].size):
        qm, qbr, _, _, _, mask, Q, K, V = _gather(layout, br, s, q, k, v, qb, kb, vb, dtype)
        for h in range(Hq):
            g = h // G
            S = (Q[:, h] @ K[:, g].T) * dtype(sc)
            l_, P = _masked_softmax(S, mask)
            O = P @ V[:, g]
            o[qm, h], lse[qm, h] = O[: qm.size], l_[: qm.size]
            if qbr.size:
                ob[qbr, h], lseb[qbr, h] = O[qm.size:], l_[qm.size:]
    return o, lse, ob, lseb


def attn_bwd(layout, br, q, k, v, qb, kb, vb, do, dob, scale=None, dtype=np.float32):
    """Closed-form backward of ``attn_fwd`` (P recomputed, Delta from the
    oracle's own O). Returns (dq, dk, dv, dqb, dkb, dvb); dk/dv have the
    [C, N_loc, Hkv, D] layout of k/v and hold this rank's contribution."""
    N, Hq, D = q.shape
    C, Nl, Hkv, _ = k.shape
    G = Hq // Hkv
    sc = _scale(D, scale)
    nb = br["n_branch"]
    dq = np.zeros((N, Hq, D), dtype)
    dk = np.zeros((C, Nl, Hkv, D), dtype)
    dv = np.zeros((C, Nl, Hkv, D), dtype)
    dqb = np.zeros((nb, Hq, D), dtype)
    dkb = np.zeros((nb, Hkv, D), dtype)
    dvb = np.zeros((nb, Hkv, D), dtype)
    for s in range(layout["L"].size):
        qm, qbr, ksh, krow, kbr, mask, Q, K, V = _gather(layout, br, s, q, k, v, qb, kb, vb, dtype)
        dO = do[qm].astype(dtype)
        if qbr.size:
            dO = np.concatenate([dO, dob[qbr].astype(dtype)], axis=0)
        nkm = ksh.size
        for h in range(Hq):
            g = h // G
            S = (Q[:, h] @ K[:, g].T) * dtype(sc)
            _, P = _masked_softmax(S, mask)
            O = P @ V[:, g]
            delta = np.sum(dO[:, h] * O, axis=-1, keepdims=True)
            dV = P.T @ dO[:, h]
            dP = dO[:, h] @ V[:, g].T
            dS = P * (dP - delta)
            dQ = (dS @ K[:, g]) * dtype(sc)
            dK = (dS.T @ Q[:, h]) * dtype(sc)
            dq[qm, h] = dQ[: qm.size]
            if qbr.size:
                dqb[qbr, h] = dQ[qm.size:]
                dkb[kbr, g] += dK[nkm:]
                dvb[kbr, g] += dV[nkm:]
            dk[ksh, krow, g] += dK[:nkm]
            dv[ksh, krow, g] += dV[:nkm]
    return dq, dk, dv, dqb, dkb, dvb


def merge_eq2(o1, l1, o2, l2):
    """Online-softmax merge of two normalised partials (rainbus analysis, core
    method, Eq. 2). ``o*`` [..., D], ``l*`` [...]; a partial with LSE = -inf
    has weight 0, and two empty partials merge to (0, -inf)."""
    l1 = np.asarray(l1)
    l2 = np.asarray(l2)
    hi = np.maximum(l1, l2)
    empty = ~np.isfinite(hi)
    hi_safe = np.where(empty, 0.0, hi)
    e1 = np.where(np.isfinite(l1), np.exp(np.where(np.isfinite(l1), l1, 0.0) - hi_safe), 0.0)
    e2 = np.where(np.isfinite(l2), np.exp(np.where(np.isfinite(l2), l2, 0.0) - hi_safe), 0.0)
    tot = e1 + e2
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, hi_safe + np.log(np.where(empty, 1.0, tot)))
    w1 = np.where(empty, 0.0, e1 / np.where(empty, 1.0, tot))
    w2 = np.where(empty, 0.0, e2 / np.where(empty, 1.0, tot))
    return w1[..., None] * o1 + w2[..., None] * o2, lse


def attn_fwd_split(layout, br, q, k, v, qb=None, kb=None, vb=None, scale=None,
                   dtype=np.float32, return_partials=False):
    """The split form: for ring step i = 0..C-1 a partial over the main keys of
    shard (r - i) mod C only, then the branch-local partial over the anchor's
    own branch keys, every partial merged into the running result by Eq. 2
    (ai.info summary, Methodology; rainbus analysis, method steps, step two).
    Returns (o, lse, ob, lseb) like ``attn_fwd``; with ``return_partials`` also
    the list of per-step partials and the branch partial."""
    N, Hq, D = q.shape
    C = layout["C"]
    r = layout["r"]
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = _scale(D, scale)
    nb = br["n_branch"]
    acc_o = np.zeros((N, Hq, D), dtype)
    acc_l = np.full((N, Hq), -np.inf, dtype)
    acc_ob = np.zeros((nb, Hq, D), dtype)
    acc_lb = np.full((nb, Hq), -np.inf, dtype)
    steps = []
    problems = [_gather(layout, br, s, q, k, v, qb, kb, vb, dtype) for s in range(layout["L"].size)]

    def partial(select):
        po = np.zeros((N, Hq, D), dtype)
        pl = np.full((N, Hq), -np.inf, dtype)
        pob = np.zeros((nb, Hq, D), dtype)
        plb = np.full((nb, Hq), -np.inf, dtype)
        for (qm, qbr, ksh, krow, kbr, mask, Q, K, V) in problems:
            keep = np.zeros(mask.shape[1], dtype=bool)
            keep[: ksh.size] = select(ksh, None)
            keep[ksh.size:] = select(None, kbr)
            m = mask & keep[None, :]
            for h in range(Hq):
                g = h // G
                S = (Q[:, h] @ K[:, g].T) * dtype(sc)
                l_, P = _masked_softmax(S, m)
                O = P @ V[:, g]
                po[qm, h], pl[qm, h] = O[: qm.size], l_[: qm.size]
                if qbr.size:
                    pob[qbr, h], plb[qbr, h] = O[qm.size:], l_[qm.size:]
        return po, pl, pob, plb

    for i in range(C):
        shard = (r - i) % C
        po, pl, pob, plb = partial(lambda ksh, kbr, sh=shard: (ksh == sh) if ksh is not None else np.zeros(kbr.size, bool))
        steps.append((shard, po, pl, pob, plb))
        acc_o, acc_l = merge_eq2(acc_o, acc_l, po, pl)
        acc_ob, acc_lb = merge_eq2(acc_ob, acc_lb, pob, plb)
    _, _, bob, blb = partial(lambda ksh, kbr: np.zeros(ksh.size, bool) if ksh is not None else np.ones(kbr.size, bool))
    out_ob, out_lb = merge_eq2(acc_ob, acc_lb, bob, blb)
    res = (acc_o.astype(dtype), acc_l.astype(dtype), out_ob.astype(dtype), out_lb.astype(dtype))
    if return_partials:
        return res + (steps, (bob, blb))
    return res


# ---------------------------------------------------------------------------
# Row-sampled evaluation for workloads too large for the dense form.


class SeqKeys:
    """Main keys of one sequence gathered into position order (real positions
    only), in ``dtype``; shared by every sampled row of that sequence."""

    def __init__(self, layout, s, k, v, dtype):
        sh, row = _seq_main_key_index(layout, s)
        self.shard, self.row = sh, row
        self.K = k[sh, row].astype(dtype)
        self.V = v[sh, row].astype(dtype)


def attn_rows(layout, br, q, k, v, qb, kb, vb, main_rows=(), branch_rows=(),
              scale=None, dtype=np.float32, do=None, dob=None, seq_keys=None,
              dk_acc=None, dv_acc=None):
    """Forward (and with ``do``/``dob`` the backward share) of selected rows
    only, each against its own visible key set, following the same
    definitions as ``attn_fwd``/``attn_bwd``.

    Returns a dict with 'o', 'lse' (and 'dq') per selected main row and per
    selected branch row. If ``dk_acc``/``dv_acc`` dicts are given, the
    selected rows' contributions to the main-key gradients are accumulated
    into them per sequence ([L_s, Hkv, D] arrays, position order)."""
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = dtype(_scale(D, scale))
    kind = br["kind"]
    want_bwd = do is not None
    cache = {} if seq_keys is None else seq_keys

    def keys_for(s):
        if s not in cache:
            cache[s] = SeqKeys(layout, s, k, v, dtype)
        return cache[s]

    out = {"main": {}, "branch": {}}
    jobs = []
    for row in main_rows:
        jobs.append(("main", int(row)))
    for row in branch_rows:
        jobs.append(("branch", int(row)))
    for kind_row, row in jobs:
        if kind_row == "main":
            s = int(layout["seq"][row])
            if layout["is_pad"][row]:
                res = dict(o=np.zeros((Hq, D), dtype), lse=np.full(Hq, -np.inf, dtype))
                if want_bwd:
                    res["dq"] = np.zeros((Hq, D), dtype)
                out["main"][row] = res
                continue
            bound = int(layout["pos"][row])
            qv = q[row].astype(dtype)
            dov = do[row].astype(dtype) if want_bwd else None
            bkeys = np.zeros(0, np.int64)
        else:
            a = int(br["b_anchor"][row])
            s = int(br["anchor_seq"][a])
            bound = int(br["anchor_pos"][a])
            qv = qb[row].astype(dtype)
            dov = dob[row].astype(dtype) if want_bwd else None
            lo, hi = int(br["branch_off"][a]), int(br["branch_off"][a + 1])
            js = np.arange(hi - lo)
            if kind == _pack.KIND_BLOCK_BIDIR:
                bkeys = lo + js
            else:
                bkeys = lo + js[js <= br["b_j"][row]]
        sk = keys_for(s)
        n = bound + 1
        res = dict(o=np.zeros((Hq, D), dtype), lse=np.zeros(Hq, dtype))
        if want_bwd:
            res["dq"] = np.zeros((Hq, D), dtype)
        for g in range(Hkv):
            Kg = sk.K[:n, g]
            Vg = sk.V[:n, g]
            if bkeys.size:
                Kg = np.concatenate([Kg, kb[bkeys, g].astype(dtype)], axis=0)
                Vg = np.concatenate([Vg, vb[bkeys, g].astype(dtype)], axis=0)
            Qg = qv[g * G:(g + 1) * G]
            S = (Qg @ Kg.T) * sc
            m = np.max(S, axis=-1, keepdims=True)
            e = np.exp(S - m)
            tot = np.sum(e, axis=-1, keepdims=True)
            P = e / tot
            O = P @ Vg
            res["o"][g * G:(g + 1) * G] = O
            res["lse"][g * G:(g + 1) * G] = (m + np.log(tot))[:, 0]
            if want_bwd:
                dOg = dov[g * G:(g + 1) * G]
                delta = np.sum(dOg * O, axis=-1, keepdims=True)
                dP = dOg @ Vg.T
                dS = P * (dP - delta)
                res["dq"][g * G:(g + 1) * G] = (dS @ Kg) * sc
                if dk_acc is not None:
                    if s not in dk_acc:
                        dk_acc[s] = np.zeros((sk.K.shape[0], Hkv, D), dtype)
                        dv_acc[s] = np.zeros((sk.K.shape[0], Hkv, D), dtype)
                    dk_acc[s][:n, g] += (dS[:, :n].T @ Qg) * sc
                    dv_acc[s][:n, g] += P[:, :n].T @ dOg
        out[kind_row][row] = res
    return out


# ---------------------------------------------------------------------------
# A subset of a rank's rows in the dense masked form.


def attn_subset(layout, br, q, k, v, qb, kb, vb, main_rows=(), anchors=(), do=None, dob=None,
                scale=None, dtype=np.float32, row_block=512):
    """Dense masked forward (and with ``do``/``dob`` the backward) of a subset
    of the rank's rows: the given main rows and every branch row of the given
    local anchors, each against its whole visible key set, by the definitions
    of ``attn_fwd``/``attn_bwd``. The key list of a sequence holds its main
    keys at positions 0 .. (largest bound among the selected rows) and the
    branch keys of the selected anchors; keys beyond it are seen by none of
    the selected rows. Rows are taken in blocks of ``row_block``.

    Returns a dict: 'main_rows', 'branch_rows' (the row indices, in the order
    of the outputs), 'o', 'lse', 'dq' [len(main_rows), Hq, D], 'ob', 'lseb',
    'dqb' for the branch rows, and the subset's contributions to the key
    gradients 'dk', 'dv' [C, N_loc, Hkv, D] and 'dkb', 'dvb' [N_b, Hkv, D].
    Pad rows get O = 0 and LSE = -inf."""
    N, Hq, D = q.shape
    C, Nl, Hkv, _ = k.shape
    G = Hq // Hkv
    sc = dtype(_scale(D, scale))
    kind = br["kind"]
    want_bwd = do is not None
    main_rows = np.asarray(main_rows, np.int64)
    anchors = np.asarray(anchors, np.int64)
    branch_rows = (np.concatenate([np.arange(br["branch_off"][a], br["branch_off"][a + 1])
                                   for a in anchors]).astype(np.int64)
                   if anchors.size else np.zeros(0, np.int64))
    res = {"main_rows": main_rows, "branch_rows": branch_rows,
           "o": np.zeros((main_rows.size, Hq, D), dtype),
           "lse": np.full((main_rows.size, Hq), -np.inf, dtype),
           "ob": np.zeros((branch_rows.size, Hq, D), dtype),
           "lseb": np.full((branch_rows.size, Hq), -np.inf, dtype)}
    if want_bwd:
        res.update(dq=np.zeros((main_rows.size, Hq, D), dtype),
                   dqb=np.zeros((branch_rows.size, Hq, D), dtype),
                   dk=np.zeros((C, Nl, Hkv, D), dtype), dv=np.zeros((C, Nl, Hkv, D), dtype),
                   dkb=np.zeros((br["n_branch"], Hkv, D), dtype),
                   dvb=np.zeros((br["n_branch"], Hkv, D), dtype))
    # output slot of every selected row: main rows first, then branch rows
    for s in range(layout["L"].size):
        mi = np.nonzero((layout["seq"][main_rows] == s) & (layout["is_pad"][main_rows] == 0))[0]
        bi = np.nonzero(br["anchor_seq"][br["b_anchor"][branch_rows]] == s)[0] \
            if branch_rows.size else np.zeros(0, np.int64)
        if mi.size + bi.size == 0:
            continue
        qrows_m = main_rows[mi]
        qrows_b = branch_rows[bi]
        bounds = np.concatenate([layout["pos"][qrows_m],
                                 br["anchor_pos"][br["b_anchor"][qrows_b]]]).astype(np.int64)
        n_main = int(bounds.max()) + 1
        shard_of, row_of = _seq_main_key_index(layout, s)
        ksh, krow = shard_of[:n_main], row_of[:n_main]
        kbr = qrows_b  # branch keys are stored row-for-row with branch queries
        Q = np.concatenate([q[qrows_m].astype(dtype), qb[qrows_b].astype(dtype)], axis=0)
        K = np.concatenate([k[ksh, krow].astype(dtype), kb[kbr].astype(dtype)], axis=0)
        V = np.concatenate([v[ksh, krow].astype(dtype), vb[kbr].astype(dtype)], axis=0)
        if want_bwd:
            dO = np.concatenate([do[qrows_m].astype(dtype), dob[qrows_b].astype(dtype)], axis=0)
        key_pos = np.arange(n_main)
        # per query: its bound, and for branch rows its anchor and step
        q_is_branch = np.concatenate([np.zeros(qrows_m.size, bool), np.ones(qrows_b.size, bool)])
        q_anchor = np.concatenate([np.full(qrows_m.size, -1), br["b_anchor"][qrows_b]])
        q_j = np.concatenate([np.full(qrows_m.size, -1), br["b_j"][qrows_b]])
        k_anchor = br["b_anchor"][kbr]
        k_j = br["b_j"][kbr]
        nq = Q.shape[0]
        for r0 in range(0, nq, row_block):
            r1 = min(nq, r0 + row_block)
            mask = np.zeros((r1 - r0, n_main + kbr.size), dtype=bool)
            for i in range(r0, r1):
                mask[i - r0, :n_main] = key_pos <= bounds[i]
                if q_is_branch[i]:
                    same = k_anchor == q_anchor[i]
                    if kind == _pack.KIND_BLOCK_BIDIR:
                        vis = same
                    else:
                        vis = same & (k_j <= q_j[i])
                    mask[i - r0, n_main:] = vis
            for h in range(Hq):
                g = h // G
                S = (Q[r0:r1, h] @ K[:, g].T) * sc
                l_, P = _masked_softmax(S, mask)
                O = P @ V[:, g]
                for i in range(r0, r1):
                    slot_o, slot_l = (("o", "lse") if not q_is_branch[i] else ("ob", "lseb"))
                    j = mi[i] if not q_is_branch[i] else bi[i - qrows_m.size]
                    res[slot_o][j, h] = O[i - r0]
                    res[slot_l][j, h] = l_[i - r0]
                if not want_bwd:
                    continue
                dOh = dO[r0:r1, h]
                delta = np.sum(dOh * O, axis=-1, keepdims=True)
                dP = dOh @ V[:, g].T
                dS = P * (dP - delta)
                dQ = (dS @ K[:, g]) * sc
                dK = (dS.T @ Q[r0:r1, h]) * sc
                dV = P.T @ dOh
                for i in range(r0, r1):
                    if not q_is_branch[i]:
                        res["dq"][mi[i], h] = dQ[i - r0]
                    else:
                        res["dqb"][bi[i - qrows_m.size], h] = dQ[i - r0]
                res["dk"][ksh, krow, g] += dK[:n_main]
                res["dv"][ksh, krow, g] += dV[:n_main]
                res["dkb"][kbr, g] += dK[n_main:]
                res["dvb"][kbr, g] += dV[n_main:]
    return res
