"""Every CP rank of a workload stitched back into the full batch (test
infrastructure). A workload's inputs are drawn once in global form; each
rank's local inputs are gathered from them; a runner computes one rank; its
outputs go back to their global rows through the zigzag permutation, the
partial dK/dV of every main key are summed over ranks, and the result is
compared with the oracle on the whole batch as one rank (C = 1)."""

import time

import numpy as np

import workloads
from oracle import pack

from helpers import grad_ok, lse_err, max_abs, oracle_grouped, oracle_structs, rel_l2, say


class GlobalBatch:
    """Inputs of a workload in global form: main rows by (sequence, position)
    in packed real order, branch rows by (global anchor, step). Every rank's
    local inputs, and the full batch's, are gathered from these, so the ranks
    of one workload see one consistent set of tensors."""

    def __init__(self, w, seed):
        self.w = w
        self.lens = np.asarray(w.seqlens, np.int64)
        self.cu = np.concatenate([[0], np.cumsum(self.lens)])
        n_real = int(self.cu[-1])
        if w.kind == pack.KIND_TTT:
            self.anchors = np.arange(n_real)
            blens = np.full(n_real, w.depth_or_block, np.int64)
        else:
            self.anchors = np.asarray(w.anchors, np.int64)
            blens = (np.asarray(w.branch_lens, np.int64) if w.branch_lens is not None
                     else np.full(self.anchors.size, w.depth_or_block, np.int64))
        self.boff = np.concatenate([[0], np.cumsum(blens)])
        nb = int(self.boff[-1])
        rng = np.random.default_rng(seed)

        def draw(rows, heads):
            x = rng.standard_normal((rows, heads, w.d), dtype=np.float32)
            return workloads.f32_to_bf16_bits(x)

        self.t = {"q": draw(n_real, w.hq), "k": draw(n_real, w.hkv), "v": draw(n_real, w.hkv),
                  "qb": draw(nb, w.hq), "kb": draw(nb, w.hkv), "vb": draw(nb, w.hkv),
                  "do": draw(n_real, w.hq), "dob": draw(nb, w.hq)}

    def main_index(self, lay):
        """Global real index of every local main row (-1 for pads)."""
        idx = self.cu[lay["seq"]] + lay["pos"]
        return np.where(lay["is_pad"] == 1, -1, idx)

    def branch_index(self, br):
        """Global branch row of every local branch row."""
        a = br["b_anchor"]
        gpos = self.cu[br["anchor_seq"][a]] + br["anchor_pos"][a]
        ga = np.searchsorted(self.anchors, gpos)
        assert np.array_equal(self.anchors[ga], gpos)
        return self.boff[ga] + br["b_j"]

    def rank_inputs(self, lay, br):
        C = lay["C"]
        mi = self.main_index(lay)
        bi = self.branch_index(br)

        def rows(name, idx):
            src = self.t[name]
            out = np.zeros((idx.size,) + src.shape[1:], src.dtype)
            ok = idx >= 0
            out[ok] = src[idx[ok]]
            return out

        shards = [self.main_index(pack.zigzag_layout(list(self.lens), C, s)) for s in range(C)]
        raw = {"q": rows("q", mi), "do": rows("do", mi),
               "k": np.stack([rows("k", sh) for sh in shards]),
               "v": np.stack([rows("v", sh) for sh in shards]),
               "qb": self.t["qb"][bi], "kb": self.t["kb"][bi], "vb": self.t["vb"][bi],
               "dob": self.t["dob"][bi]}
        return raw, mi, bi, shards



def _fwd_ok(name, go, wo, gl, wl):
    e_o, r_o, e_l = max_abs(go, wo), rel_l2(go, wo), lse_err(gl, wl)
    say(f"  {name}: max|dO|={e_o:.3e} relL2={r_o:.3e} max|dLSE|={e_l:.3e}")
    return e_o, r_o, e_l


def stitch_and_compare(w, run_rank, seed, oracle_threads=4):
    """Run ``run_rank(wr, lay, br, raw)`` for every rank r of workload ``w``
    (it returns host float32 arrays o, lse, ob, lseb, dq, dk, dv, dqb, dkb,
    dvb for the rank's local rows), stitch, and return the comparison errors
    against the full-batch oracle: {name: (max-abs, rel-L2[, max |dLSE|])}."""
    gb = GlobalBatch(w, seed=seed)
    n_real, nb = int(gb.cu[-1]), int(gb.boff[-1])
    say(f"[case] stitch {w.name}: {len(w.seqlens)} seqs, {n_real} tokens, {nb} branch rows, C={w.C}")
    st = {k: np.zeros((n_real, w.hq) + ((w.d,) if k in ("o", "dq") else ()), np.float32)
          for k in ("o", "lse", "dq")}
    stb = {k: np.zeros((nb, w.hq) + ((w.d,) if k in ("ob", "dqb") else ()), np.float32)
           for k in ("ob", "lseb", "dqb")}
    dkg = np.zeros((n_real, w.hkv, w.d), np.float32)
    dvg = np.zeros_like(dkg)
    dkbg = np.zeros((nb, w.hkv, w.d), np.float32)
    dvbg = np.zeros_like(dkbg)
    seen_b = np.zeros(nb, np.int64)
    for r in range(w.C):
        wr = workloads.Workload(f"{w.name}-r{r}", w.seqlens, w.C, r, w.kind, w.depth_or_block,
                                w.hq, w.hkv, w.d, w.dtype, True, w.seed, anchors=w.anchors,
                                branch_lens=w.branch_lens)
        lay, br = oracle_structs(wr)
        raw, mi, bi, shards = gb.rank_inputs(lay, br)
        res = run_rank(wr, lay, br, raw)
        real = mi >= 0
        assert np.all(np.isneginf(res["lse"][~real])), "pad rows must have LSE = -inf"
        assert np.all(res["o"][~real] == 0), "pad rows must have O = 0"
        st["o"][mi[real]] = res["o"][real]
        st["lse"][mi[real]] = res["lse"][real]
        st["dq"][mi[real]] = res["dq"][real]
        if bi.size:
            stb["ob"][bi] = res["ob"]
            stb["lseb"][bi] = res["lseb"]
            stb["dqb"][bi] = res["dqb"]
            dkbg[bi] += res["dkb"]
            dvbg[bi] += res["dvb"]
            seen_b[bi] += 1
        for s, sh in enumerate(shards):
            ok = sh >= 0
            np.add.at(dkg, sh[ok], res["dk"][s][ok])
            np.add.at(dvg, sh[ok], res["dv"][s][ok])
            assert np.all(res["dk"][s][~ok] == 0) and np.all(res["dv"][s][~ok] == 0), \
                "pad keys carry gradient"
        say(f"  rank {r}: {lay['n_local']} rows, {br['n_branch']} branch rows")
    assert np.all(seen_b == 1), "every anchor must belong to exactly one rank"
    w1 = workloads.Workload(f"{w.name}-c1", w.seqlens, 1, 0, w.kind, w.depth_or_block, w.hq,
                            w.hkv, w.d, w.dtype, True, w.seed, anchors=w.anchors,
                            branch_lens=w.branch_lens)
    lay1, br1 = oracle_structs(w1)
    raw1, mi1, bi1, shards1 = gb.rank_inputs(lay1, br1)
    dec = {k: workloads.as_f32(w1, v) for k, v in raw1.items()}
    t0 = time.time()
    ref = oracle_grouped(lay1, br1, *(dec[k] for k in ("q", "k", "v", "qb", "kb", "vb")),
                         dec["do"], dec["dob"], threads=oracle_threads, log=say)
    say(f"  full-batch oracle done in {time.time() - t0:.0f} s")
    real1 = mi1 >= 0
    wo = np.zeros_like(st["o"])
    wl = np.zeros_like(st["lse"])
    wq = np.zeros_like(st["dq"])
    wo[mi1[real1]], wl[mi1[real1]], wq[mi1[real1]] = (ref["o"][real1], ref["lse"][real1],
                                                      ref["dq"][real1])
    wk = np.zeros_like(dkg)
    wv = np.zeros_like(dvg)
    wk[shards1[0][real1]] = ref["dk"][0][real1]
    wv[shards1[0][real1]] = ref["dv"][0][real1]
    out = {"o": _fwd_ok("o (stitched)", st["o"], wo, st["lse"], wl)}
    pairs = [("dq (stitched)", st["dq"], wq), ("dk (sum over ranks)", dkg, wk),
             ("dv (sum over ranks)", dvg, wv)]
    if nb:
        wob = np.zeros_like(stb["ob"])
        wlb = np.zeros_like(stb["lseb"])
        wqb = np.zeros_like(stb["dqb"])
        wkb = np.zeros_like(dkbg)
        wvb = np.zeros_like(dvbg)
        wob[bi1], wlb[bi1], wqb[bi1] = ref["ob"], ref["lseb"], ref["dqb"]
        wkb[bi1], wvb[bi1] = ref["dkb"], ref["dvb"]
        out["ob"] = _fwd_ok("ob (stitched)", stb["ob"], wob, stb["lseb"], wlb)
        pairs += [("dqb (stitched)", stb["dqb"], wqb), ("dkb (stitched)", dkbg, wkb),
                  ("dvb (stitched)", dvbg, wvb)]
    for name, got, want in pairs:
        _, ma, rl = grad_ok(got, want, True)
        ref_inf = float(np.max(np.abs(want))) if want.size else 0.0
        say(f"  {name}: max-abs={ma:.3e} relL2={rl:.3e} |ref|inf={ref_inf:.3e}")
        out[name.split()[0]] = (ma, rl, ref_inf)
    return out
