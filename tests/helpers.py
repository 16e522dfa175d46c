"""Shared helpers of the GPU tests: building a workload's plan and inputs on
both sides (oracle on the host, HIP library on the device) and the error
measures the tolerances are stated in."""

import sys

import numpy as np

import workloads
from oracle import attn, pack


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_structs(w):
    lay = pack.zigzag_layout(w.seqlens, w.C, w.r)
    if w.kind == pack.KIND_TTT:
        br = pack.branch_index(lay, w.kind, w.depth_or_block)
    elif w.kind == pack.KIND_NONE:
        br = pack.branch_index(lay, w.kind)
    else:
        br = pack.branch_index(lay, w.kind, w.depth_or_block, w.anchors, w.branch_lens)
    return lay, br


def make_plan(ba, w):
    p = ba.Plan(w.seqlens, w.C, w.r, w.kind, w.depth_or_block, w.anchors, w.branch_lens,
                w.hq, w.hkv, w.d, w.dtype)
    return p.upload()


def to_device(torch, w, arr):
    if w.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def to_host(t):
    if t is None:
        return None
    return t.float().cpu().numpy()


def inputs(w, n_local, n_branch, names=workloads.TENSOR_ORDER):
    """Host inputs (encoded) and their float32 decoding for the oracle."""
    raw = workloads.draw(w, n_local, n_branch, names=names)
    dec = {k: workloads.as_f32(w, v) for k, v in raw.items()}
    return raw, dec


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def lse_err(got, want):
    """max |got - want| over finite entries; infinities must match exactly."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), "LSE infinities differ"
    assert np.all(got[~fin] == want[~fin]), "LSE infinities differ in sign"
    return float(np.max(np.abs(got[fin] - want[fin]))) if fin.any() else 0.0


def grad_ok(got, want, bf16):
    """Gradient tolerance: bf16 inputs: max-abs <= 2e-2 * max(1, |ref|_inf) and
    relative L2 <= 1e-2; fp32 inputs: max-abs <= 1e-4 * max(1, |ref|_inf)."""
    if np.asarray(want).size == 0:
        return True, 0.0, 0.0
    ma = max_abs(got, want)
    ref = float(np.max(np.abs(want)))
    rl = rel_l2(got, want)
    if bf16:
        return (ma <= 2e-2 * max(1.0, ref) and rl <= 1e-2), ma, rl
    return ma <= 1e-4 * max(1.0, ref), ma, rl


__all__ = ["attn", "pack", "workloads"]


class LazyF32:
    """Row access to an encoded input array, decoded to float32 on indexing
    (for the row-sampled oracle on full-size workloads)."""

    def __init__(self, w, raw):
        self.w, self.raw, self.shape = w, raw, raw.shape

    def __getitem__(self, idx):
        return workloads.as_f32(self.w, self.raw[idx])
