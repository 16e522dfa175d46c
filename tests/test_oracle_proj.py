"""Pins of the oracle's draft-layer projection (oracle/proj.py), CPU only:
pure-Python loops on tiny inputs, properties that fix rotary embedding
(rotation of each (i, i + d/2) pair, identity at position 0, dot products
that depend only on the position difference), the RMS norm's unit output RMS,
and the row positions by brute force over the branch index."""

import math

import numpy as np
import pytest

from oracle import pack, proj


def _loops_project(x, w, hq, hkv, d, pos, theta, qn, kn, eps):
    """The same definition in plain Python loops."""
    rows, hidden = len(x), len(x[0])
    nout = (hq + 2 * hkv) * d
    y = [[sum(x[r][t] * w[c][t] for t in range(hidden)) for c in range(nout)] for r in range(rows)]

    def heads(r, first, n):
        return [y[r][(first + h) * d:(first + h + 1) * d] for h in range(n)]

    def norm(vec, wt):
        ms = sum(a * a for a in vec) / d
        return [a / math.sqrt(ms + eps) * wt[i] for i, a in enumerate(vec)]

    def rot(vec, p):
        half = d // 2
        out = list(vec)
        for i in range(half):
            ang = p * theta ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = vec[i] * c - vec[i + half] * s
            out[i + half] = vec[i + half] * c + vec[i] * s
        return out

    q, k, v = [], [], []
    for r in range(rows):
        q.append([rot(norm(hv, qn), pos[r]) for hv in heads(r, 0, hq)])
        k.append([rot(norm(hv, kn), pos[r]) for hv in heads(r, hq, hkv)])
        v.append(heads(r, hq + hkv, hkv))
    return np.array(q), np.array(k), np.array(v)


def test_projection_matches_plain_loops():
    rng = np.random.default_rng(0)
    hq, hkv, d, hidden, rows = 4, 2, 8, 6, 5
    x = rng.standard_normal((rows, hidden))
    w = rng.standard_normal(((hq + 2 * hkv) * d, hidden))
    qn = rng.standard_normal(d)
    kn = rng.standard_normal(d)
    pos = np.array([0, 1, 7, 100, 4096])
    got = proj.project(x, w, hq, hkv, d, pos, theta=10000.0, q_norm=qn, k_norm=kn, eps=1e-6)
    want = _loops_project(x.tolist(), w.tolist(), hq, hkv, d, pos.tolist(), 10000.0, qn.tolist(),
                          kn.tolist(), 1e-6)
    for g, t in zip(got, want):
        np.testing.assert_allclose(g, t, rtol=1e-12, atol=1e-12)


def test_rope_rotates_pairs_and_is_identity_at_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 3, 16))
    pos = np.array([0, 1, 2, 50, 1000, 262143])
    y = proj.rope(x, pos, 1e6)
    np.testing.assert_allclose(y[0], x[0], atol=0)
    # each (i, i + 8) pair keeps its length
    n_x = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_y = y[..., :8] ** 2 + y[..., 8:] ** 2
    np.testing.assert_allclose(n_y, n_x, rtol=1e-12)
    # pair 0 turns by exactly the position (theta^0 = 1)
    ang = np.arctan2(y[..., 8], y[..., 0]) - np.arctan2(x[..., 8], x[..., 0])
    diff = np.angle(np.exp(1j * (ang - pos[:, None])))
    np.testing.assert_allclose(diff, 0, atol=1e-9)


def test_rope_dot_products_depend_on_the_position_difference_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    dots = []
    for m in (5, 123, 9000):
        qm = proj.rope(q, np.array([m]), 10000.0)
        kn = proj.rope(k, np.array([m - 4]), 10000.0)
        dots.append(float(np.sum(qm * kn)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


def test_rms_norm_gives_unit_rms_and_ignores_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, 128)) * 7.0
    y = proj.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(proj.rms_norm(3.0 * x, np.ones(128), 0.0), y, rtol=1e-12)


@pytest.mark.parametrize("kind", [pack.KIND_TTT, pack.KIND_BLOCK_CAUSAL])
def test_row_positions_by_brute_force(kind):
    lens, C, r = [40, 23], 2, 1
    lay = pack.zigzag_layout(lens, C, r)
    if kind == pack.KIND_TTT:
        br = pack.branch_index(lay, kind, 3)
    else:
        br = pack.branch_index(lay, kind, 0, [5, 30, 41, 60], [4, 2, 3, 5])
    np.testing.assert_array_equal(proj.row_positions(lay, br, False), lay["pos"])
    want = []
    for a in range(br["anchor_row"].size):
        n = int(br["branch_off"][a + 1] - br["branch_off"][a])
        want += [int(br["anchor_pos"][a]) + 1 + j for j in range(n)]
    np.testing.assert_array_equal(proj.row_positions(lay, br, True), want)


def test_rope_pair_angles_form_the_frequency_progression():
    # at a small position every pair turns by less than pi, so its angle is
    # readable: pair i turns by pos * theta^(-2i/d), a geometric progression
    # from pos with ratio theta^(-2/d)
    d, theta, p = 16, 500.0, 1.5
    x = np.zeros((1, 1, d))
    x[..., : d // 2] = 1.0
    y = proj.rope(x, np.array([p]), theta)
    ang = np.arctan2(y[0, 0, d // 2:], y[0, 0, : d // 2])
    np.testing.assert_allclose(ang[0], p, rtol=1e-12)
    np.testing.assert_allclose(ang[1:] / ang[:-1], theta ** (-2.0 / d), rtol=1e-12)
