"""Host logic of the library on the CPU: the C ABI loads and exports every
declared symbol; the C++ planner matches the oracle's packer and branch index
bit for bit; the kernels' work lists cover every row and key exactly once;
invalid arguments are rejected with the documented status."""

import os
import re

import numpy as np
import pytest

import workloads
from oracle import pack

ba = pytest.importorskip("branch_attention_speculative_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "branch_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:ba|branch_attn)_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = ba.lib()
    names = _declared_functions()
    assert "branch_attn_fwd" in names and "branch_attn_bwd" in names
    for n in names:
        assert hasattr(L, n), f"missing export {n}"


def _oracle(w, r=None):
    lay = pack.zigzag_layout(w.seqlens, w.C, w.r if r is None else r)
    if w.kind == pack.KIND_TTT:
        br = pack.branch_index(lay, w.kind, w.depth_or_block)
    elif w.kind == pack.KIND_NONE:
        br = pack.branch_index(lay, w.kind)
    else:
        br = pack.branch_index(lay, w.kind, w.depth_or_block, w.anchors, w.branch_lens)
    return lay, br


def _plan(w, r=None):
    return ba.Plan(w.seqlens, w.C, w.r if r is None else r, w.kind, w.depth_or_block, w.anchors,
                   w.branch_lens, w.hq, w.hkv, w.d, w.dtype)


def _compare(w, r=None):
    lay, br = _oracle(w, r)
    p = _plan(w, r)
    idx = p.indices()
    for name in ("cu_real", "cu_pad", "cu_local", "perm", "is_pad", "pos", "seq"):
        assert np.array_equal(idx[name], lay[name]), name
    for name in ("anchor_row", "anchor_pos", "anchor_seq", "branch_off"):
        assert np.array_equal(idx[name], br[name]), name
    info = p.info
    pc = pack.pair_counts(lay, br)
    assert info["n_local_rows"] == lay["n_local"]
    assert info["n_branch_rows"] == br["n_branch"]
    assert info["n_pad_rows"] == int(lay["is_pad"].sum())
    assert (info["pairs_main"], info["pairs_prefix"], info["pairs_local"], info["pairs_total"]) == \
        (pc["main"], pc["prefix"], pc["local"], pc["total"])
    return p, lay, br


@pytest.mark.parametrize("name", workloads.ALL + [n + "_r" for n in workloads.ALL if n != "tiny"])
def test_plan_matches_oracle_on_workloads(name):
    w = workloads.make(name)
    _compare(w)


def test_plan_matches_oracle_every_rank_small():
    for name in ("dflash_r", "dspark_r", "ttt32k_r"):
        w = workloads.make(name)
        for r in range(w.C):
            _compare(w, r)


@pytest.mark.parametrize("C,r", [(16, 15), (33, 7), (64, 0), (64, 63)])
def test_plan_matches_oracle_at_large_cp_degree(C, r):
    # up to the largest CP degree the planner accepts; short and long
    # sequences, so that some chunks are one row or all pads
    for kind, depth, anchors, blens in ((pack.KIND_TTT, 3, None, None),
                                        (pack.KIND_BLOCK_CAUSAL, 0, [0, 500, 1499, 1600], [4, 64, 1, 9])):
        w = workloads.Workload("bigc", [1500, 7, 2 * C + 1, 130], C, r, kind, depth, 8, 2, 128, "bf16",
                               True, 0, anchors=anchors, branch_lens=blens)
        p, lay, br = _compare(w)
        _check_worklists(p, lay, br, w)


@pytest.mark.parametrize("seed", range(12))
def test_plan_matches_oracle_random(seed):
    rng = np.random.default_rng(1000 + seed)
    C = int(rng.integers(1, 9))
    S = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(1, 400, size=S)]
    kind = int(rng.integers(0, 4))
    n_real = sum(lens)
    anchors = blens = None
    depth = int(rng.integers(1, 9))
    if kind in (2, 3):
        na = int(rng.integers(0, min(n_real, 50) + 1))
        anchors = [int(x) for x in np.sort(rng.choice(n_real, size=na, replace=False))]
        blens = [int(x) for x in rng.integers(1, 20, size=na)]
    G = int(2 ** rng.integers(0, 5))
    hkv = int(rng.integers(1, 4))
    w = workloads.Workload("rand", lens, C, int(rng.integers(0, C)), kind,
                           depth if kind != 0 else 0, hkv * G, hkv, 128, "bf16", True, 0,
                           anchors=anchors, branch_lens=blens)
    p, lay, br = _compare(w)
    _check_worklists(p, lay, br, w)


def _check_worklists(p, lay, br, w):
    G = w.hq // w.hkv
    N, NB, C = lay["n_local"], br["n_branch"], w.C
    # query tiles: every (kv-head, main row) and (kv-head, branch row) exactly once
    qt = p.worklist(0)
    seen_m = np.zeros((w.hkv, N), int)
    seen_b = np.zeros((w.hkv, NB), int)
    bound_m = np.where(lay["is_pad"] == 1, -1, lay["pos"])
    bound_b = br["anchor_pos"][br["b_anchor"]] if NB else np.zeros(0, int)
    for g, src, row0, nrows, seq_off, c, pmin, pmax in qt:
        if nrows == 0:
            continue
        assert nrows * G <= 256
        rows = np.arange(row0, row0 + nrows)
        (seen_b if src else seen_m)[g, rows] += 1
        b = (bound_b if src else bound_m)[rows]
        assert pmin == b.min() and pmax == b.max()
        seqs = (br["anchor_seq"][br["b_anchor"][rows]] if src else lay["seq"][rows])
        assert np.all(seqs == seqs[0])
        s = seqs[0]
        assert seq_off == lay["cu_local"][s] and c == lay["c"][s]
    assert np.all(seen_m == 1) and np.all(seen_b == 1)
    # key tiles: every (kv-head, shard, row) exactly once; the query range is
    # exactly the rows of the sequence that see at least one key of the tile,
    # and inside it the kernel's visibility test (key kk at position
    # kpos0 + kk) gives the true answer for every key. Tiles may span the two
    # chunks of a shard, whose true positions then jump.
    kt = p.worklist(1)
    seen_k = np.zeros((w.hkv, C, N), int)
    shard_pos = [pack.zigzag_layout(w.seqlens, C, sh)["pos"] for sh in range(C)]
    joined = 0
    packed = 0
    for g, sh, krow0, kpos0, nk, qm0, qm1, qb0, qb1, s, run, run_off in kt:
        if nk == 0:
            continue
        assert nk <= 128
        lo, hi = lay["cu_local"][s], lay["cu_local"][s + 1]
        if run == 0:  # consecutive rows of one shard
            assert run_off == 0
            shs = np.full(nk, sh)
            rows = krow0 + np.arange(nk)
        else:  # chunk pairs of consecutive shards packed back to back
            assert run == 2 * lay["c"][s] and krow0 == lo and 0 <= run_off < run
            v = run_off + np.arange(nk)
            shs = sh + v // run
            rows = krow0 + v % run
            assert shs.max() < C
            packed += 1
        assert lo <= rows.min() and rows.max() < hi
        np.add.at(seen_k, (g, shs, rows), 1)
        true_pos = np.array([shard_pos[a][b] for a, b in zip(shs, rows)])
        kern_pos = kpos0 + np.arange(nk)
        joined += int(np.any(np.diff(true_pos) != 1))
        want = [i for i in range(lo, hi) if bound_m[i] >= true_pos.min()]
        assert list(range(qm0, qm1)) == want
        bm = bound_m[qm0:qm1, None]
        assert np.array_equal(bm >= kern_pos[None], bm >= true_pos[None])
        if NB:
            in_s = np.nonzero(br["anchor_seq"][br["b_anchor"]] == s)[0]
            want_b = [i for i in in_s if bound_b[i] >= true_pos.min()]
            assert list(range(qb0, qb1)) == want_b
            bb = bound_b[qb0:qb1, None]
            assert np.array_equal(bb >= kern_pos[None], bb >= true_pos[None])
        else:
            assert qb0 == qb1
    assert np.all(seen_k == 1)
    # branch tiles: whole anchors, each exactly once per kv-head
    bt = p.worklist(2)
    A = br["anchor_row"].size
    seen_a = np.zeros((w.hkv, A), int)
    for g, a0, a1, rows in bt:
        if rows == 0:
            continue
        seen_a[g, a0:a1] += 1
        assert rows == br["branch_off"][a1] - br["branch_off"][a0]
        assert rows <= 64 and (rows * G <= 128 or a1 - a0 == 1)
    assert np.all(seen_a == 1)
    return joined, packed


@pytest.mark.parametrize("name", ["tiny", "ttt32k_r", "dflash_r", "dspark_r", "long256k_r"])
def test_worklists_cover_everything(name):
    w = workloads.make(name)
    p, lay, br = _compare(w)
    joined, packed = _check_worklists(p, lay, br, w)
    if name in ("ttt32k_r", "dspark_r"):  # short chunks: key tiles span chunks and shards
        assert joined > 0 and packed > 0


def test_xcd_interleave_keeps_kv_heads_together_on_the_long_workload():
    # 8 kv-heads of equal cost: workgroup b runs on XCD b % 8, and every XCD
    # should meet the tiles of one kv-head only
    w = workloads.make("long256k")
    p = _plan(w)
    qt = p.worklist(0)
    for x in range(8):
        heads = set(qt[x::8][qt[x::8][:, 3] > 0][:, 0].tolist())
        assert len(heads) == 1


@pytest.mark.parametrize("args,status", [
    (dict(seqlens=[], cp=2, r=0), "BA_E_INVALID"),
    (dict(seqlens=[10], cp=2, r=2), "BA_E_INVALID"),
    (dict(seqlens=[0], cp=1, r=0), "BA_E_INVALID"),
    (dict(seqlens=[10], cp=1, r=0, hq=12, hkv=8), "BA_E_INVALID"),
    (dict(seqlens=[10], cp=1, r=0, hq=24, hkv=8), "BA_E_UNSUPPORTED"),
    (dict(seqlens=[10], cp=1, r=0, d=64), "BA_E_UNSUPPORTED"),
    (dict(seqlens=[10], cp=1, r=0, kind=1, depth=0), "BA_E_INVALID"),
    (dict(seqlens=[10], cp=1, r=0, kind=1, depth=65), "BA_E_UNSUPPORTED"),
    (dict(seqlens=[10], cp=1, r=0, kind=2, depth=4, anchors=[3, 3]), "BA_E_INVALID"),
    (dict(seqlens=[10], cp=1, r=0, kind=2, depth=4, anchors=[10]), "BA_E_INVALID"),
    (dict(seqlens=[10], cp=1, r=0, kind=3, anchors=[2], blens=[65]), "BA_E_UNSUPPORTED"),
    (dict(seqlens=[10], cp=1, r=0, kind=1, depth=2, anchors=[2]), "BA_E_INVALID"),
])
def test_invalid_plans_are_rejected(args, status):
    with pytest.raises(ba.BranchAttnError, match=status):
        ba.Plan(args["seqlens"], args["cp"], args["r"], args.get("kind", 0), args.get("depth", 0),
                args.get("anchors"), args.get("blens"), args.get("hq", 32), args.get("hkv", 8),
                args.get("d", 128), "bf16")


def test_fwd_without_upload_is_rejected_before_any_device_call():
    p = ba.Plan([64], 2, 0, ba.KIND_NONE, hq=2, hkv=2, d=64, dtype="fp32")
    a = ba.FwdArgs()
    st = ba.lib().branch_attn_fwd(p.handle, a, None)
    assert ba.lib().ba_status_str(st) == b"BA_E_INVALID"
    assert b"not uploaded" in ba.lib().ba_last_error()


def test_binding_checks_the_caller_workspace():
    torch = pytest.importorskip("torch")
    cpu = torch.device("cpu")
    # the size is counted in bytes, whatever the dtype
    assert ba._workspace(torch.empty(16, dtype=torch.float32), 64, cpu) == 64
    with pytest.raises(ValueError, match="needs 65 bytes"):
        ba._workspace(torch.empty(16, dtype=torch.float32), 65, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        ba._workspace(torch.empty(8, 8, dtype=torch.uint8).t(), 1, cpu)
    with pytest.raises(ValueError, match="expected device"):
        ba._workspace(torch.empty(8, dtype=torch.uint8), 1, torch.device("cuda", 0))


def test_key_walk_choice_by_chunk_size():
    # run lists when every chunk is <= 8192 rows, segments otherwise; the
    # override forces either and returns to the automatic choice with mode 0
    ba = pytest.importorskip("branch_attention_speculative_amd")
    short = ba.Plan([5000, 3000], 4, 0, 1, 2, hq=8, hkv=2, d=128, dtype="bf16")
    assert short.info["run_walk"] == 1
    long_ = ba.Plan([262144], 8, 0, 1, 2, hq=8, hkv=2, d=128, dtype="bf16")
    assert long_.info["run_walk"] == 0  # chunks of 16384 rows
    edge = ba.Plan([8192 * 16], 8, 0, 0, 0, hq=8, hkv=2, d=128, dtype="bf16")
    assert edge.info["run_walk"] == 1  # exactly 8192-row chunks
    long_.set_walk("runs")
    assert long_.info["run_walk"] == 1
    short.set_walk("segments")
    assert short.info["run_walk"] == 0
    short.set_walk("auto")
    assert short.info["run_walk"] == 1
    with pytest.raises(ba.BranchAttnError):
        ba.lib()
        _ = ba._check(ba.lib().ba_plan_set_walk(short.handle, 3), "ba_plan_set_walk")
