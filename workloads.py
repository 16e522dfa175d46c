"""Seeded synthetic workloads for draft branch attention.

This module only draws inputs: sequence lengths, anchor positions, branch
lengths and N(0,1) tensors, plus the float32 -> bfloat16 round-to-nearest-even
encoding of those draws. It holds none of the attention arithmetic and none
of the packing logic, and it serves both the oracle side (tests, CPU
baseline) and the GPU side (tests, bench) with identical inputs.

Workloads (standing in for the pages' operator benchmarks: EAGLE-3 TTT and
DFlash/DSpark block drafts at fixed global lengths up to 256K, packed
variable-length batches; ai.info summary, Main Findings; rainbus analysis,
Figs. 5 and 6). The RL datasets the pages train on are not used: attention
consumes projected activations, which are stood in for by N(0,1) draws.

  tiny     1 x 256 tokens, C=2, 2/2 heads, D=64, fp32, TTT depth 3, fwd
  ttt32k   4 sequences U[4096,12288] summing to 32768, C=4, 32/8/128 bf16,
           TTT depth 7, fwd
  dflash   8 sequences summing to 65536 (uniform composition), C=4, 32/8/128
           bf16, 1024 anchors, bidirectional blocks of 16, fwd+bwd
  long256k 1 x 262144 tokens, C=8, 32/8/128 bf16, TTT depth 7, fwd+bwd
  dspark   log-uniform [1024,8192] lengths summing to 131072, C=8, 64/4/128
           bf16, 2048 anchors, causal blocks of 8 or 16 (p=0.5), fwd+bwd

Reduced variants (suffix ``_r``) keep the head configuration, kind, C and
structure but shrink the token count so the dense oracle finishes in seconds.
``long256k_r16k`` is the larger reduction of the long workload: 1 x 16384
tokens, C=8 (chunks of 1024 rows, several key tiles each), 32/8/128 bf16,
TTT depth 7, fwd+bwd.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

KIND_NONE, KIND_TTT, KIND_BLOCK_BIDIR, KIND_BLOCK_CAUSAL = 0, 1, 2, 3
KIND_NAMES = {KIND_NONE: "none", KIND_TTT: "ttt", KIND_BLOCK_BIDIR: "block_bidir",
              KIND_BLOCK_CAUSAL: "block_causal"}


@dataclass
class Workload:
    name: str
    seqlens: List[int]
    C: int
    r: int
    kind: int
    depth_or_block: int
    hq: int
    hkv: int
    d: int
    dtype: str                      # "bf16", "fp32" or "fp8" (fp8 E4M3 q/k/qb/kb, bf16 rest)
    bwd: bool
    seed: int
    anchors: Optional[List[int]] = None
    branch_lens: Optional[List[int]] = None
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_real(self):
        return int(sum(self.seqlens))


# ---------------------------------------------------------------------------
# structure generators


def lengths_uniform_fixed_total(rng, n, lo, hi, total):
    """n lengths in [lo, hi] summing to ``total``: draw n-1 uniformly, set the
    last to the remainder, redraw until it falls in range."""
    while True:
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return [int(x) for x in head] + [last]


def lengths_uniform_composition(rng, n, total, quantum=8):
    """Uniform random composition of ``total`` into n parts: n-1 distinct cut
    points drawn from the multiples of ``quantum`` strictly inside (0, total)."""
    cuts = rng.choice(np.arange(quantum, total, quantum), size=n - 1, replace=False)
    cuts = np.sort(cuts)
    edges = np.concatenate([[0], cuts, [total]])
    return [int(x) for x in np.diff(edges)]


def lengths_log_uniform(rng, lo, hi, total):
    """Lengths round(exp(U(ln lo, ln hi))) until the running total reaches
    ``total``; the last one is truncated to hit the total exactly."""
    out = []
    acc = 0
    while acc < total:
        x = int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))
        x = min(x, total - acc)
        out.append(x)
        acc += x
    return out


def anchors_uniform(rng, n_real, n_anchors):
    """Anchors uniform without replacement over the real tokens of the packed
    batch, sorted."""
    return [int(x) for x in np.sort(rng.choice(n_real, size=n_anchors, replace=False))]


# ---------------------------------------------------------------------------
# workloads


def make(name):
    """Build a named workload (structure only; tensors come from ``draw``)."""
    if name == "long256k_r16k":
        return Workload(name, [16384], 8, 0, KIND_TTT, 7, 32, 8, 128, "bf16", True, 4)
    base = name[:-2] if name.endswith("_r") else name
    reduced = name.endswith("_r")
    seed = {"tiny": 1, "ttt32k": 2, "dflash": 3, "long256k": 4, "dspark": 5}[base]
    rng = np.random.default_rng(seed)
    if base == "tiny":
        return Workload(name, [256], 2, 0, KIND_TTT, 3, 2, 2, 64, "fp32", False, seed)
    if base == "ttt32k":
        if reduced:
            lens = lengths_uniform_fixed_total(rng, 4, 300, 1500, 3300)
        else:
            lens = lengths_uniform_fixed_total(rng, 4, 4096, 12288, 32768)
        return Workload(name, lens, 4, 0, KIND_TTT, 7, 32, 8, 128, "bf16", False, seed)
    if base == "dflash":
        total, n_anch = (4096, 64) if reduced else (65536, 1024)
        lens = lengths_uniform_composition(rng, 8, total)
        anchors = anchors_uniform(rng, total, n_anch)
        return Workload(name, lens, 4, 0, KIND_BLOCK_BIDIR, 16, 32, 8, 128, "bf16", True,
                        seed, anchors=anchors)
    if base == "long256k":
        n = 2048 if reduced else 262144
        return Workload(name, [n], 8, 0, KIND_TTT, 7, 32, 8, 128, "bf16", True, seed)
    if base == "dspark":
        if reduced:
            lens = lengths_log_uniform(rng, 64, 512, 3000)
            n_anch = 96
        else:
            lens = lengths_log_uniform(rng, 1024, 8192, 131072)
            n_anch = 2048
        total = int(sum(lens))
        anchors = anchors_uniform(rng, total, n_anch)
        blens = [int(x) for x in np.where(rng.random(n_anch) < 0.5, 8, 16)]
        return Workload(name, lens, 8, 0, KIND_BLOCK_CAUSAL, 16, 64, 4, 128, "bf16", True,
                        seed, anchors=anchors, branch_lens=blens)
    raise KeyError(name)


ALL = ["tiny", "ttt32k", "dflash", "long256k", "dspark"]


# ---------------------------------------------------------------------------
# tensors


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs here are finite normal draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_table():
    """Values of the 127 non-negative finite OCP fp8 E4M3 codes 0x00..0x7E
    (exponent bias 7, subnormals at exponent field 0, no infinities, 0x7F is
    NaN), in code order, which is also increasing value order."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3 = _e4m3_table()
E4M3_MAX = float(_E4M3[-1])  # 448


def f32_to_e4m3_bits(x):
    """float32 -> OCP fp8 E4M3 codes (uint8), round to nearest, ties to the
    even code; magnitudes beyond 448 saturate to 448. Inputs are finite."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 126)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x) & (code != 0), code | 0x80, code).astype(np.uint8)


def e4m3_bits_to_f32(b):
    b = np.asarray(b, dtype=np.uint8)
    mag = _E4M3[np.minimum(b & 0x7F, 126)].astype(np.float32)
    return np.where(b & 0x80, -mag, mag).astype(np.float32)


TENSOR_ORDER = ["q", "k", "v", "qb", "kb", "vb", "do", "dob"]
# tensors that an fp8 workload holds in fp8 E4M3 (the score operands); the
# others stay bf16
FP8_TENSORS = ("q", "k", "qb", "kb")


def tensor_shapes(n_local, n_branch, C, hq, hkv, d):
    return {
        "q": (n_local, hq, d), "k": (C, n_local, hkv, d), "v": (C, n_local, hkv, d),
        "qb": (n_branch, hq, d), "kb": (n_branch, hkv, d), "vb": (n_branch, hkv, d),
        "do": (n_local, hq, d), "dob": (n_branch, hq, d),
    }


def _fill(w, tensor_id, shape, lo, n, out, chunk):
    rng = np.random.default_rng([w.seed, 1000 + tensor_id, lo // chunk])
    x = rng.standard_normal(n, dtype=np.float32)
    if out.dtype == np.uint8:
        out[lo:lo + n] = f32_to_e4m3_bits(x)
    elif w.dtype in ("bf16", "fp8"):
        out[lo:lo + n] = f32_to_bf16_bits(x)
    else:
        out[lo:lo + n] = x


def draw(w, n_local, n_branch, names=TENSOR_ORDER, chunk=1 << 22, threads=None):
    """Draw the workload's tensors: N(0,1) float32, encoded as bf16 bit
    patterns (uint16) for bf16 workloads or kept float32. Element block b of
    tensor t (blocks of ``chunk`` elements) comes from its own generator seeded
    by (seed, 1000 + t, b), so the values do not depend on which tensors are
    requested or on how many threads draw them. ``n_local`` and ``n_branch``
    are the row counts of the packed local share and of the local branch rows."""
    import concurrent.futures
    import os
    shapes = tensor_shapes(n_local, n_branch, w.C, w.hq, w.hkv, w.d)
    out = {}
    jobs = []
    for t, nm in enumerate(TENSOR_ORDER):
        if nm not in names:
            continue
        shp = shapes[nm]
        n = int(np.prod(shp))
        if w.dtype == "fp8" and nm in FP8_TENSORS:
            buf = np.empty(n, np.uint8)
        else:
            buf = np.empty(n, np.uint16 if w.dtype in ("bf16", "fp8") else np.float32)
        out[nm] = buf
        for lo in range(0, n, chunk):
            jobs.append((t, shp, lo, min(chunk, n - lo), buf))
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda j: _fill(w, j[0], j[1], j[2], j[3], j[4], chunk), jobs))
    return {nm: out[nm].reshape(shapes[nm]) for nm in out}


def as_f32(w, arr):
    """Decode a drawn tensor to float32 values: fp8 E4M3 codes (uint8) and
    bf16 bit patterns (uint16) are widened exactly, float32 is kept."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint8:
        return e4m3_bits_to_f32(arr)
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr)
    return np.asarray(arr, np.float32)
