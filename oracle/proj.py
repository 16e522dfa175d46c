"""Oracle: the draft layer step that produces the attention inputs -- Q/K/V
projections of the draft's hidden states, a per-head RMS norm of Q and K,
and rotary position embedding at each row's position (test infrastructure
only).

What the pages fix (arXiv:2609.07108):

* paperlens walkthrough, "The two walls": EAGLE-3's training-time test feeds
  its own predictions back and rehearses several steps ahead, so a branch
  grows from every position; DFlash emits a whole block in one pass.
* rainbus analysis, background on the three draft families, and method
  steps, step four: EAGLE-3 feeds the previous step's hidden state back as
  the next step's input (one TTT pass per step); DFlash produces the whole
  block at once; DSpark adds a Markov head on top.

What they leave open, and the readings taken here (the Qwen3-style draft
layer the workloads are shaped after):

* projection: y = x W^T with W in [(hq + 2 hkv) d, hidden] (q heads, then k
  heads, then v heads);
* per-head RMS norm of q and k over d with a learned weight, before RoPE;
* RoPE in the rotate-half form: dims i and i + d/2 (i < d/2) turn by
  pos * theta^(-2i/d);
* positions: a main row sits at its position in the sequence; branch row j
  of the anchor at position p stands for the token j + 1 steps after the
  anchor and sits at p + 1 + j (TTT step j, block slot j).

Parity: pinned in tests/test_oracle_proj.py (pure-Python loops on tiny
inputs, RoPE's norm preservation and relative-position property, the RMS
norm's unit output RMS, positions by brute force over the branch index).
"""

import numpy as np


def row_positions(layout, br, branch):
    """Position of every local main row (branch=False; pads keep their padded
    position) or of every local branch row (branch=True)."""
    if not branch:
        return np.asarray(layout["pos"], np.int64)
    a = br["b_anchor"]
    return (br["anchor_pos"][a] + 1 + br["b_j"]).astype(np.int64)


def rms_norm(x, w, eps):
    """x / sqrt(mean(x^2 over the last axis) + eps) * w."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope(x, pos, theta):
    """Rotate-half rotary embedding of x [..., rows, heads, d] at positions
    pos [rows]: for i < d/2, (x_i, x_{i+d/2}) turns by pos * theta^(-2i/d)."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]  # [rows, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def project(x, w, hq, hkv, d, pos, theta=0.0, q_norm=None, k_norm=None, eps=1e-6):
    """Q, K, V of rows x [rows, hidden] (float64): y = x W^T split into heads;
    q and k RMS-normed per head when the weights are given, then rotated by
    RoPE at ``pos`` when theta > 0. Returns (q [rows,hq,d], k [rows,hkv,d],
    v [rows,hkv,d])."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    y = x @ w.T
    n = x.shape[0]
    q = y[:, :hq * d].reshape(n, hq, d)
    k = y[:, hq * d:(hq + hkv) * d].reshape(n, hkv, d)
    v = y[:, (hq + hkv) * d:].reshape(n, hkv, d)
    if q_norm is not None:
        q = rms_norm(q, q_norm, eps)
    if k_norm is not None:
        k = rms_norm(k, k_norm, eps)
    if theta > 0:
        q = rope(q, pos, theta)
        k = rope(k, pos, theta)
    return q, k, v
