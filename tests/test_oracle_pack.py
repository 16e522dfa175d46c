"""Pins of the oracle's packer and branch index (CPU only).

Each test checks the oracle against something other than itself: the layout
the tiny workload states, the permutation property, closed-form pair counts,
and the per-ring-step balance that zigzag sharding exists for (rainbus
analysis of arXiv:2609.07108, background section on context parallelism).
"""

import os

import numpy as np
import pytest

from oracle import pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden_layout():
    out = {}
    with open(os.path.join(GOLDEN, "zigzag_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rank, span = line.split()
            lo, hi = (int(x) for x in span.split("-"))
            out.setdefault(int(rank), []).extend(range(lo, hi + 1))
    return out


def test_tiny_layout_matches_golden():
    gold = _read_golden_layout()
    for r in (0, 1):
        lay = pack.zigzag_layout([256], 2, r)
        assert lay["n_local"] == 128
        assert list(lay["pos"]) == gold[r]
        assert not lay["is_pad"].any()


@pytest.mark.parametrize("seed", range(6))
def test_union_of_ranks_is_a_bijection(seed):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 9))
    S = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(1, 300, size=S)]
    seen = []
    for r in range(C):
        lay = pack.zigzag_layout(lens, C, r)
        assert lay["n_local"] * C == lay["cu_pad"][-1]
        seen.append(lay["perm"])
        # pads are exactly the positions at or past the real length
        assert np.array_equal(lay["is_pad"], (lay["pos"] >= np.asarray(lens)[lay["seq"]]).astype(int))
        # padded lengths are the smallest multiples of 2C that fit
        assert np.all(lay["P"] % (2 * C) == 0) and np.all(lay["P"] - lay["L"] < 2 * C)
    allp = np.sort(np.concatenate(seen))
    assert np.array_equal(allp, np.arange(int(sum(pack.zigzag_layout(lens, C, 0)["P"]))))


@pytest.mark.parametrize("C,c", [(1, 5), (2, 64), (4, 7), (8, 16)])
def test_single_sequence_main_pairs_closed_form(C, c):
    # a rank holding chunks r and 2C-1-r of a pad-free sequence sees
    # c^2 (2C-1) + c(c+1) = 2Cc^2 + c causal pairs, the same on every rank
    for r in range(C):
        lay = pack.zigzag_layout([2 * C * c], C, r)
        br = pack.branch_index(lay, pack.KIND_NONE)
        assert pack.pair_counts(lay, br)["main"] == 2 * C * c * c + c


def test_tiny_workload_pair_counts():
    lay = pack.zigzag_layout([256], 2, 0)
    br = pack.branch_index(lay, pack.KIND_TTT, 3)
    pc = pack.pair_counts(lay, br)
    # main: sum of (p+1) over p in 0..63 and 192..255
    main = sum(p + 1 for p in range(64)) + sum(p + 1 for p in range(192, 256))
    assert pc["main"] == main == 16448
    assert pc["prefix"] == 3 * main           # three chained rows per anchor
    assert pc["local"] == 128 * (1 + 2 + 3)   # row j sees branch keys 0..j
    assert br["n_branch"] == 384


@pytest.mark.parametrize("seed", range(5))
def test_anchors_land_on_exactly_one_rank(seed):
    rng = np.random.default_rng(100 + seed)
    C = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(1, 200, size=int(rng.integers(1, 5)))]
    n_real = sum(lens)
    na = int(rng.integers(1, min(n_real, 40) + 1))
    anchors = np.sort(rng.choice(n_real, size=na, replace=False))
    blens = rng.integers(1, 6, size=na)
    cu = np.concatenate([[0], np.cumsum(lens)])
    got = []
    for r in range(C):
        lay = pack.zigzag_layout(lens, C, r)
        br = pack.branch_index(lay, pack.KIND_BLOCK_CAUSAL, 0, anchors, blens)
        for a in range(br["anchor_row"].size):
            row = br["anchor_row"][a]
            # the anchor's main row really is that sequence position and not a pad
            assert lay["seq"][row] == br["anchor_seq"][a]
            assert lay["pos"][row] == br["anchor_pos"][a]
            assert not lay["is_pad"][row]
            g = cu[br["anchor_seq"][a]] + br["anchor_pos"][a]
            got.append(g)
            assert br["branch_off"][a + 1] - br["branch_off"][a] == blens[np.searchsorted(anchors, g)]
        # local anchors are ordered by local main row
        assert np.all(np.diff(br["anchor_row"]) > 0)
    assert sorted(got) == list(anchors)


def test_ttt_every_real_position_is_an_anchor():
    lens = [37, 5, 64]
    C = 3
    total = 0
    for r in range(C):
        lay = pack.zigzag_layout(lens, C, r)
        br = pack.branch_index(lay, pack.KIND_TTT, 2)
        real_rows = np.nonzero(lay["is_pad"] == 0)[0]
        assert np.array_equal(br["anchor_row"], real_rows)
        assert br["n_branch"] == 2 * real_rows.size
        assert np.array_equal(br["b_j"], np.tile([0, 1], real_rows.size))
        total += real_rows.size
    assert total == sum(lens)


def test_invalid_inputs_raise():
    with pytest.raises(ValueError):
        pack.zigzag_layout([], 2, 0)
    with pytest.raises(ValueError):
        pack.zigzag_layout([10], 2, 2)
    lay = pack.zigzag_layout([10], 1, 0)
    with pytest.raises(ValueError):
        pack.branch_index(lay, pack.KIND_BLOCK_BIDIR, 4, [3, 3])
    with pytest.raises(ValueError):
        pack.branch_index(lay, pack.KIND_BLOCK_BIDIR, 4, [10])
    with pytest.raises(ValueError):
        pack.branch_index(lay, pack.KIND_TTT, 0)
