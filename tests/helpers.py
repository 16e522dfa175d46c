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
    """Encoded host input -> device tensor of the library's element type:
    uint8 fp8 E4M3 codes -> float8_e4m3fn, uint16 bf16 bits -> bfloat16,
    float32 kept."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint8:
        t = torch.from_numpy(arr).view(torch.float8_e4m3fn)
    elif arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
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


def shift_late_keys(lam):
    """Input preparation: add lam * u (u a fixed unit vector) to every main key
    in the second half of its sequence. A query's scores against those keys
    move by lam * scale * <q, u> together: for queries with <q, u> > 0 they
    jump far above the scores of earlier keys, for <q, u> < 0 they fall far
    below them. Inside each half the attention stays as diffuse as with plain
    N(0, 1) data. Keys that share a large component are also the input domain
    where a bf16 backward loses accuracy (the rounding errors of dS and Delta
    are multiplied by that component in dQ = scale dS K)."""
    def prep(w, lay, raw):
        k = workloads.as_f32(w, raw["k"]).copy()
        u = np.random.default_rng(99).standard_normal(w.d).astype(np.float32)
        u /= np.linalg.norm(u)
        for s_ in range(w.C):
            ls = pack.zigzag_layout(w.seqlens, w.C, s_)
            late = ls["pos"] >= (ls["L"][ls["seq"]] + 1) // 2
            k[s_][late] += lam * u
        raw["k"] = workloads.f32_to_bf16_bits(k) if w.dtype == "bf16" else k
    return prep


def random_workload(seed, dtype="bf16"):
    """A seeded random small workload: the branch kinds in turn, C from 1 to
    16 and any rank, one to five sequences of 1..1200 tokens, GQA groups of 1
    to 16 over 1 to 4 kv-heads, TTT depths 1..8, block anchors anywhere in the
    packed stream with block lengths 1..64. The fp8 form has no backward
    flag (its tests call the backward themselves)."""
    rng = np.random.default_rng(7000 + seed)
    kind = [pack.KIND_NONE, pack.KIND_TTT, pack.KIND_BLOCK_BIDIR, pack.KIND_BLOCK_CAUSAL][seed % 4]
    C = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    r = int(rng.integers(0, C))
    lens = [int(x) for x in rng.integers(1, 1201, size=int(rng.integers(1, 6)))]
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8, 16]))
    depth, anchors, blens = 0, None, None
    if kind == pack.KIND_TTT:
        depth = int(rng.integers(1, 9))
    elif kind != pack.KIND_NONE:
        total = sum(lens)
        n_a = int(rng.integers(1, min(total, 24) + 1))
        anchors = sorted(int(x) for x in rng.choice(total, size=n_a, replace=False))
        blens = [int(x) for x in rng.integers(1, 65, size=n_a)]
    name = f"random-{seed}"
    return workloads.Workload(name, lens, C, r, kind, depth, hq, hkv, 128, dtype, dtype == "bf16",
                              sum(ord(ch) for ch in name), anchors=anchors, branch_lens=blens)


def oracle_grouped(lay, br, q, k, v, qb, kb, vb, do=None, dob=None, dtype=np.float32,
                   threads=4, log=None):
    """The oracle's dense forward (and with do/dob its backward), evaluated one
    kv-group at a time on a thread pool: the oracle's heads are independent,
    and a group's q-heads see only that group's K/V, so calling it on the
    group's slices gives exactly its full-tensor result. Returns a dict with
    o, lse, ob, lseb (and dq, dk, dv, dqb, dkb, dvb)."""
    import concurrent.futures
    Hq, Hkv = q.shape[1], k.shape[2]
    G = Hq // Hkv
    want_bwd = do is not None

    def one(g):
        hs = slice(g * G, (g + 1) * G)
        gs = slice(g, g + 1)
        ins = (q[:, hs], k[:, :, gs], v[:, :, gs], qb[:, hs], kb[:, gs], vb[:, gs])
        res = dict(zip(("o", "lse", "ob", "lseb"), attn.attn_fwd(lay, br, *ins, dtype=dtype)))
        if want_bwd:
            res.update(zip(("dq", "dk", "dv", "dqb", "dkb", "dvb"),
                           attn.attn_bwd(lay, br, *ins, do[:, hs], dob[:, hs], dtype=dtype)))
        if log is not None:
            log(f"  oracle kv-group {g} done")
        return g, res

    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = dict(ex.map(one, range(Hkv)))
    out = {}
    for name in parts[0]:
        axis = {"dk": 2, "dv": 2, "dkb": 1, "dvb": 1}.get(name, 1)
        out[name] = np.concatenate([parts[g][name] for g in range(Hkv)], axis=axis)
    return out


class HeadSlice:
    """Row access to an input whose head axis (second to last) is restricted
    to ``hs``: indexing gathers the rows first, then slices the heads, so
    encoded full-size inputs are decoded only where they are read."""

    def __init__(self, arr, hs):
        self.arr, self.hs = arr, hs
        shp = list(arr.shape)
        shp[-2] = len(range(*hs.indices(shp[-2])))
        self.shape = tuple(shp)

    def __getitem__(self, idx):
        return self.arr[idx][..., self.hs, :]


def subset_grouped(lay, br, q, k, v, qb, kb, vb, main_rows, anchors, do=None, dob=None,
                   threads=8, log=None):
    """``attn.attn_subset`` evaluated one kv-group at a time on a thread pool
    (heads are independent; a group's q-heads see only its K/V). Inputs may be
    any row-indexable arrays (LazyF32 for encoded full-size tensors)."""
    import concurrent.futures
    Hq, Hkv = q.shape[1], k.shape[2]
    G = Hq // Hkv
    want_bwd = do is not None

    def one(g):
        hs, gs = slice(g * G, (g + 1) * G), slice(g, g + 1)
        r = attn.attn_subset(lay, br, HeadSlice(q, hs), HeadSlice(k, gs), HeadSlice(v, gs),
                             HeadSlice(qb, hs), HeadSlice(kb, gs), HeadSlice(vb, gs),
                             main_rows=main_rows, anchors=anchors,
                             do=HeadSlice(do, hs) if want_bwd else None,
                             dob=HeadSlice(dob, hs) if want_bwd else None)
        if log is not None:
            log(f"  oracle kv-group {g} done")
        return g, r

    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = dict(ex.map(one, range(Hkv)))
    out = {"main_rows": parts[0]["main_rows"], "branch_rows": parts[0]["branch_rows"]}
    for name in parts[0]:
        if name in out:
            continue
        axis = {"dk": 2, "dv": 2, "dkb": 1, "dvb": 1}.get(name, 1)
        out[name] = np.concatenate([parts[g][name] for g in range(Hkv)], axis=axis)
    return out


def complete_keys(lay, br, main_rows, anchors):
    """Main keys (per sequence, positions >= p*) and branch keys whose every
    viewer among the rank's rows is in the subset, so that the subset's dK/dV
    contributions are their whole gradient. Returns (boolean mask over
    [C, N_loc] shard rows, boolean mask over branch rows)."""
    C = lay["C"]
    sel_m = np.zeros(lay["n_local"], bool)
    sel_m[np.asarray(main_rows, np.int64)] = True
    A = br["anchor_row"].size
    sel_a = np.zeros(A, bool)
    sel_a[np.asarray(anchors, np.int64)] = True
    S = lay["L"].size
    pstar = np.zeros(S, np.int64)
    for i in np.nonzero(~sel_m & (lay["is_pad"] == 0))[0]:
        s = lay["seq"][i]
        pstar[s] = max(pstar[s], lay["pos"][i] + 1)
    for a in np.nonzero(~sel_a)[0]:
        s = br["anchor_seq"][a]
        pstar[s] = max(pstar[s], br["anchor_pos"][a] + 1)
    keys = np.zeros((C, lay["n_local"]), bool)
    for sh in range(C):
        ls = pack.zigzag_layout(lay["L"].tolist(), C, sh)
        keys[sh] = (ls["is_pad"] == 0) & (ls["pos"] >= pstar[ls["seq"]])
    bkeys = sel_a[br["b_anchor"]] if br["n_branch"] else np.zeros(0, bool)
    return keys, bkeys
