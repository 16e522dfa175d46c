"""Pins of the oracle's attention, backward and split form (CPU only).

Nothing here re-derives the oracle's own vectorised code: the pins are a
pure-Python brute force over the unpermuted batch (every rank stitched back),
torch's scaled-dot-product attention on plain causal cases, closed forms
(K = 0 gives LSE = ln|V(q)|; one-hot values expose the exact visible set),
central finite differences for every gradient, the gradient sum rules, and
the float32-vs-float64 bound.
"""

import math

import numpy as np
import pytest

from oracle import attn, pack

KINDS = [pack.KIND_TTT, pack.KIND_BLOCK_BIDIR, pack.KIND_BLOCK_CAUSAL, pack.KIND_NONE]


# ---------------------------------------------------------------------------
# a small problem stated in global (unpermuted) form


class Problem:
    """Global inputs: per sequence Q/K/V in position order, per anchor its
    branch Q/K/V. Anchors are (sequence, position, length)."""

    def __init__(self, seed, lens, C, kind, depth=2, n_anchors=3, hq=2, hkv=1, d=4,
                 anchor_list=None, blens=None):
        rng = np.random.default_rng(seed)
        self.lens, self.C, self.kind = list(lens), C, kind
        self.hq, self.hkv, self.d, self.G = hq, hkv, d, hq // hkv
        n_real = sum(lens)
        cu = np.concatenate([[0], np.cumsum(lens)])
        if kind == pack.KIND_TTT:
            glob = np.arange(n_real)
            blens = np.full(n_real, depth)
        elif kind == pack.KIND_NONE:
            glob = np.zeros(0, np.int64)
            blens = np.zeros(0, np.int64)
        else:
            glob = (np.sort(rng.choice(n_real, size=min(n_anchors, n_real), replace=False))
                    if anchor_list is None else np.asarray(anchor_list))
            blens = rng.integers(1, 4, size=glob.size) if blens is None else np.asarray(blens)
        self.glob_anchors, self.blens = glob, blens
        self.anchors = []
        for g, n in zip(glob, blens):
            s = int(np.searchsorted(cu, g, side="right") - 1)
            self.anchors.append((s, int(g - cu[s]), int(n)))
        self.Q = [rng.standard_normal((L, hq, d)) for L in lens]
        self.K = [rng.standard_normal((L, hkv, d)) for L in lens]
        self.V = [rng.standard_normal((L, hkv, d)) for L in lens]
        self.QB = [rng.standard_normal((n, hq, d)) for (_, _, n) in self.anchors]
        self.KB = [rng.standard_normal((n, hkv, d)) for (_, _, n) in self.anchors]
        self.VB = [rng.standard_normal((n, hkv, d)) for (_, _, n) in self.anchors]
        self.garbage = rng  # for pad rows

    # rank-local row rule, stated here independently of the oracle's packer:
    # every sequence is cut into 2C equal chunks after padding to a multiple
    # of 2C; rank rr holds chunk rr then chunk 2C-1-rr
    def local_rows(self, rr):
        rows = []
        C = self.C
        for s, L in enumerate(self.lens):
            P = -(-L // (2 * C)) * 2 * C
            c = P // (2 * C)
            for p in list(range(rr * c, (rr + 1) * c)) + list(range((2 * C - 1 - rr) * c, (2 * C - rr) * c)):
                rows.append((s, p if p < L else None))
        return rows

    def local_anchor_ids(self, rr):
        rows = self.local_rows(rr)
        index = {(s, p): i for i, (s, p) in enumerate(rows) if p is not None}
        ids = [a for a, (s, p, n) in enumerate(self.anchors) if (s, p) in index]
        return sorted(ids, key=lambda a: index[(self.anchors[a][0], self.anchors[a][1])])

    def rank_inputs(self, rr):
        """q, k, v, qb, kb, vb in the library layout for rank rr (pad rows get
        random values that must never matter)."""
        rng = np.random.default_rng(999)
        rows = self.local_rows(rr)
        n = len(rows)
        q = np.empty((n, self.hq, self.d))
        for i, (s, p) in enumerate(rows):
            q[i] = self.Q[s][p] if p is not None else rng.standard_normal((self.hq, self.d)) * 50
        k = np.empty((self.C, n, self.hkv, self.d))
        v = np.empty((self.C, n, self.hkv, self.d))
        for sh in range(self.C):
            for i, (s, p) in enumerate(self.local_rows(sh)):
                if p is None:
                    k[sh, i] = rng.standard_normal((self.hkv, self.d)) * 50
                    v[sh, i] = rng.standard_normal((self.hkv, self.d)) * 50
                else:
                    k[sh, i], v[sh, i] = self.K[s][p], self.V[s][p]
        ids = self.local_anchor_ids(rr)
        cat = lambda xs, h: (np.concatenate([xs[a] for a in ids]) if ids else np.zeros((0, h, self.d)))
        return q, k, v, cat(self.QB, self.hq), cat(self.KB, self.hkv), cat(self.VB, self.hkv)

    def oracle_structs(self, rr):
        lay = pack.zigzag_layout(self.lens, self.C, rr)
        if self.kind == pack.KIND_TTT:
            br = pack.branch_index(lay, self.kind, int(self.blens[0]))
        elif self.kind == pack.KIND_NONE:
            br = pack.branch_index(lay, self.kind)
        else:
            br = pack.branch_index(lay, self.kind, 0, self.glob_anchors, self.blens)
        return lay, br


def brute_force(pb, scale):
    """Pure-Python float64 attention over the unpermuted batch, straight from
    the visibility rules."""
    def one(qvec, keys):
        sc = [scale * sum(qvec[i] * kk[i] for i in range(pb.d)) for kk, _ in keys]
        m = max(sc)
        z = sum(math.exp(x - m) for x in sc)
        lse = m + math.log(z)
        o = [sum(math.exp(x - lse) * vv[i] for x, (_, vv) in zip(sc, keys)) for i in range(pb.d)]
        return o, lse

    O, LSE = {}, {}
    for s, L in enumerate(pb.lens):
        for p in range(L):
            for h in range(pb.hq):
                g = h // pb.G
                keys = [(pb.K[s][t][g], pb.V[s][t][g]) for t in range(p + 1)]
                O[("m", s, p, h)], LSE[("m", s, p, h)] = one(pb.Q[s][p][h], keys)
    for a, (s, pa, n) in enumerate(pb.anchors):
        for j in range(n):
            for h in range(pb.hq):
                g = h // pb.G
                keys = [(pb.K[s][t][g], pb.V[s][t][g]) for t in range(pa + 1)]
                for jj in range(n):
                    if pb.kind == pack.KIND_BLOCK_BIDIR or jj <= j:
                        keys.append((pb.KB[a][jj][g], pb.VB[a][jj][g]))
                O[("b", a, j, h)], LSE[("b", a, j, h)] = one(pb.QB[a][j][h], keys)
    return O, LSE


CASES = [
    # (lens, C, kind, depth)
    ([7, 12], 2, pack.KIND_TTT, 2),
    ([9], 3, pack.KIND_TTT, 3),
    ([5, 11, 3], 2, pack.KIND_BLOCK_BIDIR, 0),
    ([13, 4], 3, pack.KIND_BLOCK_CAUSAL, 0),
    ([6, 10], 1, pack.KIND_BLOCK_CAUSAL, 0),
    ([8, 3], 2, pack.KIND_NONE, 0),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_brute_force_every_rank(ci):
    lens, C, kind, depth = CASES[ci]
    pb = Problem(10 + ci, lens, C, kind, depth=depth, n_anchors=4)
    scale = 0.7
    O, LSE = brute_force(pb, scale)
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        q, k, v, qb, kb, vb = pb.rank_inputs(rr)
        o, lse, ob, lseb = attn.attn_fwd(lay, br, q, k, v, qb, kb, vb, scale=scale, dtype=np.float64)
        for i, (s, p) in enumerate(pb.local_rows(rr)):
            for h in range(pb.hq):
                if p is None:
                    assert np.all(o[i, h] == 0) and lse[i, h] == -np.inf
                else:
                    np.testing.assert_allclose(o[i, h], O[("m", s, p, h)], rtol=0, atol=1e-12)
                    assert abs(lse[i, h] - LSE[("m", s, p, h)]) < 1e-12
        ids = pb.local_anchor_ids(rr)
        row = 0
        for a in ids:
            for j in range(pb.anchors[a][2]):
                for h in range(pb.hq):
                    np.testing.assert_allclose(ob[row, h], O[("b", a, j, h)], rtol=0, atol=1e-12)
                    assert abs(lseb[row, h] - LSE[("b", a, j, h)]) < 1e-12
                row += 1
        assert row == ob.shape[0]


@pytest.mark.parametrize("C", [1, 2, 4])
def test_no_branches_equals_torch_causal_sdpa(C):
    torch = pytest.importorskip("torch")
    pb = Problem(3, [21, 9, 16], C, pack.KIND_NONE, hq=4, hkv=2, d=8)
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        q, k, v, qb, kb, vb = pb.rank_inputs(rr)
        o, lse, _, _ = attn.attn_fwd(lay, br, q, k, v, qb, kb, vb, dtype=np.float64)
        for s, L in enumerate(pb.lens):
            Q = torch.from_numpy(pb.Q[s]).transpose(0, 1)[None]
            K = torch.from_numpy(pb.K[s]).repeat_interleave(pb.G, dim=1).transpose(0, 1)[None]
            V = torch.from_numpy(pb.V[s]).repeat_interleave(pb.G, dim=1).transpose(0, 1)[None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)[0].transpose(0, 1).numpy()
            for i, (ss, p) in enumerate(pb.local_rows(rr)):
                if ss == s and p is not None:
                    np.testing.assert_allclose(o[i], ref[p], rtol=0, atol=1e-12)


def _visible_count(kind, lay, br, main_row=None, branch_row=None):
    if main_row is not None:
        return 0 if lay["is_pad"][main_row] else int(lay["pos"][main_row]) + 1
    a = br["b_anchor"][branch_row]
    n = int(br["branch_off"][a + 1] - br["branch_off"][a])
    own = n if kind == pack.KIND_BLOCK_BIDIR else int(br["b_j"][branch_row]) + 1
    return int(br["anchor_pos"][a]) + 1 + own


@pytest.mark.parametrize("kind", KINDS)
def test_zero_keys_give_log_count_and_mean(kind):
    pb = Problem(5, [14, 23], 2, kind, depth=3, n_anchors=5, hq=2, hkv=2, d=3)
    for rr in range(2):
        lay, br = pb.oracle_structs(rr)
        q, k, v, qb, kb, vb = pb.rank_inputs(rr)
        k[:] = 0.0
        kb[:] = 0.0
        o, lse, ob, lseb = attn.attn_fwd(lay, br, q, k, v, qb, kb, vb, dtype=np.float64)
        for i, (s, p) in enumerate(pb.local_rows(rr)):
            n = _visible_count(kind, lay, br, main_row=i)
            if n == 0:
                assert np.all(lse[i] == -np.inf)
                continue
            assert np.all(np.abs(lse[i] - math.log(n)) < 1e-13)
            assert np.all(np.round(np.exp(lse[i])) == n)
            np.testing.assert_allclose(o[i], np.repeat(pb.V[s][: p + 1].mean(axis=0), pb.G, axis=0), atol=1e-13)
        for b in range(ob.shape[0]):
            n = _visible_count(kind, lay, br, branch_row=b)
            assert np.all(np.abs(lseb[b] - math.log(n)) < 1e-13)


@pytest.mark.parametrize("kind", [pack.KIND_TTT, pack.KIND_BLOCK_BIDIR, pack.KIND_BLOCK_CAUSAL])
def test_one_hot_values_expose_the_visible_set(kind):
    # K = 0 and a distinct one-hot value per key: O[q] = 1/|V(q)| exactly on
    # the visible keys and 0 elsewhere
    lens, C = [10, 7], 2
    pb = Problem(8, lens, C, kind, depth=2, n_anchors=4, hq=1, hkv=1, d=1)
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        q, k, v, qb, kb, vb = pb.rank_inputs(rr)
        n_main = k.shape[1]
        nb = kb.shape[0]
        D = C * n_main + nb
        k = np.zeros((C, n_main, 1, D))
        kb = np.zeros((nb, 1, D))
        q = np.zeros((q.shape[0], 1, D))
        qb = np.zeros((nb, 1, D))
        v = np.zeros((C, n_main, 1, D))
        vb = np.zeros((nb, 1, D))
        for sh in range(C):
            for i in range(n_main):
                v[sh, i, 0, sh * n_main + i] = 1.0
        for b in range(nb):
            vb[b, 0, C * n_main + b] = 1.0
        o, lse, ob, lseb = attn.attn_fwd(lay, br, q, k, v, qb, kb, vb, dtype=np.float64)
        # expected visible sets from positions, found by scanning every shard
        shard_rows = [pb.local_rows(sh) for sh in range(C)]

        def main_keys(s, bound):
            return {sh * n_main + i for sh in range(C) for i, (ss, p) in enumerate(shard_rows[sh])
                    if ss == s and p is not None and p <= bound}

        for i, (s, p) in enumerate(pb.local_rows(rr)):
            vis = set() if p is None else main_keys(s, p)
            got = set(np.nonzero(o[i, 0])[0])
            assert got == vis
            if vis:
                assert np.allclose(o[i, 0][list(vis)], 1.0 / len(vis), atol=1e-14)
        ids = pb.local_anchor_ids(rr)
        row = 0
        for a in ids:
            s, pa, n = pb.anchors[a]
            for j in range(n):
                vis = main_keys(s, pa)
                for jj in range(n):
                    if kind == pack.KIND_BLOCK_BIDIR or jj <= j:
                        vis.add(C * n_main + row - j + jj)
                got = set(np.nonzero(ob[row, 0])[0])
                assert got == vis
                assert np.allclose(ob[row, 0][list(vis)], 1.0 / len(vis), atol=1e-14)
                row += 1


def test_block_of_one_is_the_same_for_both_block_kinds():
    lens = [15, 9]
    anchors = [2, 7, 14, 20]
    outs = []
    for kind in (pack.KIND_BLOCK_BIDIR, pack.KIND_BLOCK_CAUSAL):
        pb = Problem(21, lens, 2, kind, anchor_list=anchors, blens=[1, 1, 1, 1])
        lay, br = pb.oracle_structs(1)
        outs.append(attn.attn_fwd(lay, br, *pb.rank_inputs(1), dtype=np.float64))
    for x, y in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_split_and_merge_equals_unsplit(ci):
    lens, C, kind, depth = CASES[ci]
    pb = Problem(40 + ci, lens, C, kind, depth=depth, n_anchors=4, hq=4, hkv=2, d=6)
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        ins = pb.rank_inputs(rr)
        full = attn.attn_fwd(lay, br, *ins, dtype=np.float64)
        split = attn.attn_fwd_split(lay, br, *ins, dtype=np.float64)
        for x, y in zip(full, split):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


def test_split_steps_follow_the_ring_and_balance_work():
    # one pad-free sequence: ring step i uses shard (r - i) mod C, and the
    # main pairs per step are 2c^2 + c on step 0 and 2c^2 on the others
    C, c = 4, 3
    pb = Problem(2, [2 * C * c], C, pack.KIND_NONE, hq=1, hkv=1, d=2)
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        q, k, v, qb, kb, vb = pb.rank_inputs(rr)
        k[:] = 0.0
        *_, steps, _ = attn.attn_fwd_split(lay, br, q, k, v, qb, kb, vb, dtype=np.float64,
                                           return_partials=True)
        for i, (shard, po, pl, pob, plb) in enumerate(steps):
            assert shard == (rr - i) % C
            pairs = int(np.round(np.sum(np.exp(pl[np.isfinite(pl)]))))
            assert pairs == 2 * c * c + (c if i == 0 else 0)


def test_merge_eq2_handles_empty_partials():
    o1 = np.array([[1.0, 2.0]])
    o2 = np.array([[3.0, -1.0]])
    o, l = attn.merge_eq2(o1, np.array([0.5]), o2, np.array([-np.inf]))
    np.testing.assert_array_equal(o, o1)
    assert l[0] == 0.5
    o, l = attn.merge_eq2(o1, np.array([-np.inf]), o2, np.array([-np.inf]))
    assert np.all(o == 0) and l[0] == -np.inf
    # equal LSEs average the two partials and add ln 2
    o, l = attn.merge_eq2(o1, np.array([1.0]), o2, np.array([1.0]))
    np.testing.assert_allclose(o, [[2.0, 0.5]])
    assert abs(l[0] - (1.0 + math.log(2.0))) < 1e-15


def _loss(lay, br, ins, do, dob, scale):
    o, _, ob, _ = attn.attn_fwd(lay, br, *ins, scale=scale, dtype=np.float64)
    return float(np.sum(o * do) + np.sum(ob * dob))


@pytest.mark.parametrize("ci", [0, 2, 3, 5])
def test_backward_matches_finite_differences(ci):
    lens, C, kind, depth = CASES[ci]
    pb = Problem(60 + ci, lens, C, kind, depth=depth, n_anchors=3, hq=4, hkv=2, d=5)
    rng = np.random.default_rng(ci)
    scale = 0.6
    rr = C - 1
    lay, br = pb.oracle_structs(rr)
    ins = list(pb.rank_inputs(rr))
    do = rng.standard_normal(ins[0].shape)
    dob = rng.standard_normal(ins[3].shape)
    grads = attn.attn_bwd(lay, br, *ins, do, dob, scale=scale, dtype=np.float64)
    eps = 1e-6
    for t in range(6):
        if ins[t].size == 0:
            continue
        u = rng.standard_normal(ins[t].shape)
        plus = [x.copy() for x in ins]
        minus = [x.copy() for x in ins]
        plus[t] += eps * u
        minus[t] -= eps * u
        fd = (_loss(lay, br, plus, do, dob, scale) - _loss(lay, br, minus, do, dob, scale)) / (2 * eps)
        an = float(np.sum(grads[t] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (t, fd, an)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_gradient_sum_rules(ci):
    # softmax rows sum to 1, so sum_k dV_k = sum_q dO_q per kv-group, and
    # every dS row sums to 0, so sum_k dK_k = 0
    lens, C, kind, depth = CASES[ci]
    pb = Problem(80 + ci, lens, C, kind, depth=depth, n_anchors=4, hq=4, hkv=2, d=3)
    rng = np.random.default_rng(ci)
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        ins = pb.rank_inputs(rr)
        do = rng.standard_normal(ins[0].shape)
        dob = rng.standard_normal(ins[3].shape)
        dq, dk, dv, dqb, dkb, dvb = attn.attn_bwd(lay, br, *ins, do, dob, dtype=np.float64)
        real = lay["is_pad"] == 0
        for g in range(pb.hkv):
            hs = slice(g * pb.G, (g + 1) * pb.G)
            want = do[real][:, hs].sum(axis=(0, 1)) + dob[:, hs].sum(axis=(0, 1))
            got = dv[:, :, g].sum(axis=(0, 1)) + dvb[:, g].sum(axis=0)
            np.testing.assert_allclose(got, want, atol=1e-10)
            np.testing.assert_allclose(dk[:, :, g].sum(axis=(0, 1)) + dkb[:, g].sum(axis=0), 0, atol=1e-10)
        # pad rows and pad keys carry no gradient
        assert np.all(dq[~real] == 0)
        for sh in range(C):
            pads = pack.zigzag_layout(lens, C, sh)["is_pad"] == 1
            assert np.all(dk[sh][pads] == 0) and np.all(dv[sh][pads] == 0)


def test_rank_partial_key_gradients_sum_to_the_full_gradient():
    lens, C = [11, 6], 3
    pb = Problem(7, lens, C, pack.KIND_BLOCK_CAUSAL, n_anchors=5, hq=2, hkv=1, d=4)
    rng = np.random.default_rng(1)
    per_rank = []
    for rr in range(C):
        lay, br = pb.oracle_structs(rr)
        ins = pb.rank_inputs(rr)
        do = rng.standard_normal(ins[0].shape)
        dob = rng.standard_normal(ins[3].shape)
        per_rank.append((lay, br, list(ins), do, dob))
    total_dk = sum(attn.attn_bwd(lay, br, *ins, do, dob, dtype=np.float64)[1]
                   for lay, br, ins, do, dob in per_rank)
    k0 = per_rank[0][2][1]
    u = rng.standard_normal(k0.shape)
    eps = 1e-6

    def total_loss(kk):
        tot = 0.0
        for lay, br, ins, do, dob in per_rank:
            x = list(ins)
            x[1] = kk
            tot += _loss(lay, br, x, do, dob, None)
        return tot

    fd = (total_loss(k0 + eps * u) - total_loss(k0 - eps * u)) / (2 * eps)
    assert abs(fd - float(np.sum(total_dk * u))) < 1e-6 * max(1.0, abs(fd))


def test_float32_oracle_well_inside_the_fp32_tolerance():
    # the tiny EAGLE-3 TTT workload shape: 256 tokens, C=2, 2 heads, D=64, depth 3.
    # Scores summed over D=64 in float32 carry ~sqrt(D)*2^-24*|s| absolute
    # error, which reaches O as ~1e-6; the fp32 oracle must sit well inside
    # the 1e-5 fp32 parity tolerance, so the bound is 4e-6 (observed 1.2e-6).
    rng = np.random.default_rng(1)
    lay = pack.zigzag_layout([256], 2, 0)
    br = pack.branch_index(lay, pack.KIND_TTT, 3)
    n, nb = lay["n_local"], br["n_branch"]
    ins = [rng.standard_normal((n, 2, 64)).astype(np.float32),
           rng.standard_normal((2, n, 2, 64)).astype(np.float32),
           rng.standard_normal((2, n, 2, 64)).astype(np.float32),
           rng.standard_normal((nb, 2, 64)).astype(np.float32),
           rng.standard_normal((nb, 2, 64)).astype(np.float32),
           rng.standard_normal((nb, 2, 64)).astype(np.float32)]
    a = attn.attn_fwd(lay, br, *ins, dtype=np.float32)
    b = attn.attn_fwd(lay, br, *ins, dtype=np.float64)
    for x, y in zip(a, b):
        assert np.max(np.abs(x.astype(np.float64) - y)) <= 4e-6


@pytest.mark.parametrize("ci", [0, 2, 3])
def test_row_sampled_form_matches_dense(ci):
    lens, C, kind, depth = CASES[ci]
    pb = Problem(90 + ci, lens, C, kind, depth=depth, n_anchors=4, hq=4, hkv=2, d=6)
    rng = np.random.default_rng(ci)
    rr = 1 % C
    lay, br = pb.oracle_structs(rr)
    ins = pb.rank_inputs(rr)
    do = rng.standard_normal(ins[0].shape)
    dob = rng.standard_normal(ins[3].shape)
    o, lse, ob, lseb = attn.attn_fwd(lay, br, *ins, dtype=np.float64)
    dq, dk, dv, dqb, dkb, dvb = attn.attn_bwd(lay, br, *ins, do, dob, dtype=np.float64)
    dk_acc, dv_acc = {}, {}
    rows = attn.attn_rows(lay, br, *ins, main_rows=range(lay["n_local"]),
                          branch_rows=range(br["n_branch"]), dtype=np.float64, do=do, dob=dob,
                          dk_acc=dk_acc, dv_acc=dv_acc)
    for i, res in rows["main"].items():
        np.testing.assert_allclose(res["o"], o[i], atol=1e-12)
        np.testing.assert_array_equal(np.isfinite(res["lse"]), np.isfinite(lse[i]))
        fin = np.isfinite(lse[i])
        np.testing.assert_allclose(res["lse"][fin], lse[i][fin], atol=1e-12)
        np.testing.assert_allclose(res["dq"], dq[i], atol=1e-12)
    for i, res in rows["branch"].items():
        np.testing.assert_allclose(res["o"], ob[i], atol=1e-12)
        np.testing.assert_allclose(res["lse"], lseb[i], atol=1e-12)
        np.testing.assert_allclose(res["dq"], dqb[i], atol=1e-12)
    # the main-key gradients that the row-sampled form accumulates over every
    # row of the rank (position order per sequence) are the dense backward's
    # dK/dV of the main keys (shard, local row), read back position by position
    seen = set()
    for s in range(lay["L"].size):
        L = int(lay["L"][s])
        if L == 0:
            continue
        assert s in dk_acc, s
        for p_ in range(L):
            hits = []
            for sh in range(C):
                lay_s = pack.zigzag_layout(lens, C, sh)
                idx = np.nonzero((lay_s["seq"] == s) & (lay_s["pos"] == p_))[0]
                hits += [(sh, int(i)) for i in idx]
            assert len(hits) == 1
            sh, i = hits[0]
            seen.add((sh, i))
            np.testing.assert_allclose(dk_acc[s][p_], dk[sh, i], atol=1e-12)
            np.testing.assert_allclose(dv_acc[s][p_], dv[sh, i], atol=1e-12)
    # every other key row (pads) has no gradient in the dense form either
    for sh in range(C):
        for i in range(dk.shape[1]):
            if (sh, i) not in seen:
                assert np.all(dk[sh, i] == 0) and np.all(dv[sh, i] == 0)


@pytest.mark.parametrize("ci", [0, 1, 2, 3])
@pytest.mark.parametrize("part", [False, True])
def test_subset_form_matches_dense(ci, part):
    # attn_subset on a subset of rows equals the dense forms on those rows; its
    # key gradients are the dense backward with dO zeroed on every other row
    # (dK and dV are linear in dO), so a misplaced or missing key row shows
    lens, C, kind, depth = CASES[ci]
    pb = Problem(70 + ci, lens, C, kind, depth=depth, n_anchors=4, hq=4, hkv=2, d=6)
    rng = np.random.default_rng(ci + 10)
    rr = (ci + 1) % C
    lay, br = pb.oracle_structs(rr)
    ins = pb.rank_inputs(rr)
    do = rng.standard_normal(ins[0].shape)
    dob = rng.standard_normal(ins[3].shape)
    n, A = lay["n_local"], br["anchor_row"].size
    if part:
        mrows = np.sort(rng.choice(n, size=max(1, n // 3), replace=False))
        anch = np.sort(rng.choice(A, size=A // 2, replace=False)) if A else np.zeros(0, np.int64)
    else:
        mrows, anch = np.arange(n), np.arange(A)
    sub = attn.attn_subset(lay, br, *ins, main_rows=mrows, anchors=anch, do=do, dob=dob,
                           dtype=np.float64, row_block=5)
    o, lse, ob, lseb = attn.attn_fwd(lay, br, *ins, dtype=np.float64)
    keep_m = np.zeros(n, bool)
    keep_m[mrows] = True
    brows = sub["branch_rows"]
    keep_b = np.zeros(br["n_branch"], bool)
    keep_b[brows] = True
    assert brows.size == sum(int(br["branch_off"][a + 1] - br["branch_off"][a]) for a in anch)
    dq, dk, dv, dqb, dkb, dvb = attn.attn_bwd(lay, br, *ins, do * keep_m[:, None, None],
                                              dob * keep_b[:, None, None], dtype=np.float64)
    np.testing.assert_allclose(sub["o"], o[mrows], atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(sub["lse"]), np.isneginf(lse[mrows]))  # pads
    fin = np.isfinite(lse[mrows])
    np.testing.assert_allclose(sub["lse"][fin], lse[mrows][fin], atol=1e-12)
    np.testing.assert_allclose(sub["ob"], ob[brows], atol=1e-12)
    np.testing.assert_allclose(sub["lseb"], lseb[brows], atol=1e-12)
    np.testing.assert_allclose(sub["dq"], dq[mrows], atol=1e-12)
    np.testing.assert_allclose(sub["dqb"], dqb[brows], atol=1e-12)
    for got, want in ((sub["dk"], dk), (sub["dv"], dv), (sub["dkb"], dkb), (sub["dvb"], dvb)):
        np.testing.assert_allclose(got, want, atol=1e-12)
