"""GPU parity of the draft-layer projection (ba_qkv_project) through the C
ABI against the oracle (oracle/proj.py): q, k, v = x W^T per head, per-head
RMS norm of q and k, RoPE at each row's position, written into the
attention's main-row and branch-row layouts; TTT passes with step-major
inputs; and the chain projection -> branch attention.

Tolerance: the outputs are bf16 (relative rounding 2^-9) of fp32
accumulations; the kernel and the float64 oracle may round an element to
neighbouring bf16 values, so the bar is max-abs <= 1.5e-2 * max|ref| and
relative L2 <= 4e-3 over each output."""

import numpy as np
import pytest

import workloads
from oracle import pack, proj

from helpers import lse_err, make_plan, max_abs, oracle_grouped, oracle_structs, rel_l2, say, \
    to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import branch_attention_speculative_amd as ba
    ba.lib()
    return torch, ba


def _bf16(a):
    return workloads.f32_to_bf16_bits(np.asarray(a, np.float32))


def _weights(seed, hq, hkv, d, hidden):
    rng = np.random.default_rng(seed)
    w = _bf16(rng.standard_normal(((hq + 2 * hkv) * d, hidden)) / np.sqrt(hidden))
    qn = _bf16(1.0 + 0.1 * rng.standard_normal(d))
    kn = _bf16(1.0 + 0.1 * rng.standard_normal(d))
    return w, qn, kn


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _cmp(name, got, want):
    ma, rl = max_abs(got, want), rel_l2(got, want)
    ref = float(np.max(np.abs(want))) if want.size else 0.0
    say(f"  {name}: max-abs={ma:.3e} relL2={rl:.3e} |ref|inf={ref:.3e}")
    assert ma <= 1.5e-2 * max(ref, 1e-30) and rl <= 4e-3, (name, ma, rl)


def _case(name, lens, C, r, kind, depth, hq, hkv, anchors=None, blens=None):
    return workloads.Workload(name, lens, C, r, kind, depth, hq, hkv, 128, "bf16", False,
                              sum(ord(ch) for ch in name), anchors=anchors, branch_lens=blens)


CASES = [
    _case("proj-ttt", [150, 77], 4, 3, pack.KIND_TTT, 3, 16, 4),
    _case("proj-blocks", [300, 90], 2, 1, pack.KIND_BLOCK_CAUSAL, 0, 8, 2,
          anchors=[80, 150, 220, 330, 360], blens=[32, 17, 25, 32, 9]),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("hidden,theta,norm", [(256, 1e6, True), (320, 1e4, False), (64, 0.0, True)])
def test_projection_main_and_branch_rows(env, w, hidden, theta, norm):
    torch, ba = env
    say(f"[case] projection {w.name}: hidden={hidden} theta={theta} norm={norm}")
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    N, NB = plan.info["n_local_rows"], plan.info["n_branch_rows"]
    wb, qn, kn = _weights(hidden + 7, w.hq, w.hkv, w.d, hidden)
    rng = np.random.default_rng(hidden)
    for branch, rows in ((False, N), (True, NB)):
        x = _bf16(rng.standard_normal((rows, hidden)))
        q, k, v = ba.qkv_project(plan, _dev(torch, x), _dev(torch, wb),
                                 _dev(torch, qn) if norm else None, _dev(torch, kn) if norm else None,
                                 branch=branch, rope_theta=theta)
        torch.cuda.synchronize()
        pos = proj.row_positions(lay, br, branch)
        f = workloads.bf16_bits_to_f32
        rq, rk, rv = proj.project(f(x), f(wb), w.hq, w.hkv, w.d, pos, theta,
                                  f(qn) if norm else None, f(kn) if norm else None, 1e-6)
        real = np.ones(rows, bool) if branch else lay["is_pad"] == 0
        tag = "branch" if branch else "main"
        for nm, g, t in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
            gh = to_host(g)
            _cmp(f"{tag} {nm}", gh[real], t[real])
            assert np.all(gh[~real] == 0), "pad rows must be zero"


def test_ttt_step_passes_fill_the_branch_rows_like_one_call(env):
    """EAGLE-3's training-time test runs one pass per step: pass j takes the
    step-major hidden states of step j (one row per local anchor) and fills
    branch row j of every anchor. All passes together give exactly the
    single call over every branch row."""
    torch, ba = env
    w = CASES[0]
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    NB, A = plan.info["n_branch_rows"], plan.info["n_local_anchors"]
    hidden = 192
    wb, qn, kn = _weights(3, w.hq, w.hkv, w.d, hidden)
    x = _bf16(np.random.default_rng(4).standard_normal((NB, hidden)))
    W, QN, KN = _dev(torch, wb), _dev(torch, qn), _dev(torch, kn)
    ref = ba.qkv_project(plan, _dev(torch, x), W, QN, KN, branch=True)
    out = tuple(torch.full_like(t, 7.0) for t in ref)
    boff = br["branch_off"]
    for j in range(w.depth_or_block):
        xj = x[boff[:-1] + j]  # step-major: row a = anchor a's step-j input
        ba.qkv_project(plan, _dev(torch, xj), W, QN, KN, branch=True, step=j, out=out)
    torch.cuda.synchronize()
    assert A * w.depth_or_block == NB
    for g, t in zip(out, ref):
        assert torch.equal(g, t)
    say(f"  {w.depth_or_block} step passes bit-identical to one call over {NB} branch rows")


def test_projection_at_qwen3_8b_width(env):
    """hidden 4096 with 32/8 heads (a Qwen3-8B-shaped draft layer) on the
    reduced long workload's 2,048 main and 14,336 branch rows; the oracle
    checks every 97th row."""
    torch, ba = env
    w = workloads.make("long256k_r")
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    hidden = 4096
    wb, qn, kn = _weights(11, w.hq, w.hkv, w.d, hidden)
    W, QN, KN = _dev(torch, wb), _dev(torch, qn), _dev(torch, kn)
    rng = np.random.default_rng(12)
    f = workloads.bf16_bits_to_f32
    for branch in (False, True):
        rows = plan.info["n_branch_rows"] if branch else plan.info["n_local_rows"]
        x = _bf16(rng.standard_normal((rows, hidden)))
        q, k, v = ba.qkv_project(plan, _dev(torch, x), W, QN, KN, branch=branch)
        torch.cuda.synchronize()
        sel = np.arange(0, rows, 97)
        pos = proj.row_positions(lay, br, branch)[sel]
        rq, rk, rv = proj.project(f(x[sel]), f(wb), w.hq, w.hkv, w.d, pos, 1e6, f(qn), f(kn), 1e-6)
        for nm, g, t in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
            _cmp(f"{'branch' if branch else 'main'} {nm} (4096)", to_host(g)[sel], t)


def test_projection_feeds_branch_attention(env):
    """The chain of the draft forward: project main and branch rows, put the
    main K/V in this rank's shard (the other shards' K/V come from their own
    ranks; here drawn), run branch attention, and compare with the oracle's
    attention on the same projected values."""
    torch, ba = env
    w = workloads.Workload("proj-chain", [300, 120], 2, 1, pack.KIND_TTT, 3, 8, 2, 128, "bf16",
                           False, 77)
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    N, NB = plan.info["n_local_rows"], plan.info["n_branch_rows"]
    hidden = 256
    wb, qn, kn = _weights(5, w.hq, w.hkv, w.d, hidden)
    W, QN, KN = _dev(torch, wb), _dev(torch, qn), _dev(torch, kn)
    rng = np.random.default_rng(6)
    q, k_own, v_own = ba.qkv_project(plan, _dev(torch, _bf16(rng.standard_normal((N, hidden)))),
                                     W, QN, KN)
    qb, kb, vb = ba.qkv_project(plan, _dev(torch, _bf16(rng.standard_normal((NB, hidden)))),
                                W, QN, KN, branch=True)
    k = _dev(torch, _bf16(rng.standard_normal((w.C, N, w.hkv, w.d))))
    v = _dev(torch, _bf16(rng.standard_normal((w.C, N, w.hkv, w.d))))
    k[w.r].copy_(k_own)
    v[w.r].copy_(v_own)
    o, lse, ob, lseb = ba.fwd(plan, q, k, v, qb, kb, vb)
    torch.cuda.synchronize()
    ins = [to_host(t) for t in (q, k, v, qb, kb, vb)]
    ref = oracle_grouped(lay, br, *ins)
    for nm, go, gl, wo, wl in (("o", o, lse, ref["o"], ref["lse"]),
                               ("ob", ob, lseb, ref["ob"], ref["lseb"])):
        e_o, r_o, e_l = max_abs(to_host(go), wo), rel_l2(to_host(go), wo), lse_err(to_host(gl), wl)
        say(f"  {nm}: max|dO|={e_o:.3e} relL2={r_o:.3e} max|dLSE|={e_l:.3e}")
        assert e_o <= 2e-2 and r_o <= 1e-2 and e_l <= 1e-3


def test_projection_rejects_bad_calls(env):
    torch, ba = env
    import ctypes
    w = CASES[1]  # a block plan: no TTT step passes
    plan = make_plan(ba, w)
    L = ba.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bad = [dict(target=2, step=-1, hidden=64), dict(target=0, step=0, hidden=64),
           dict(target=1, step=0, hidden=64), dict(target=0, step=-1, hidden=96),
           dict(target=0, step=-1, hidden=64, rope_theta=float("inf"))]
    for kw in bad:
        a = ba.ProjArgs(**kw)
        assert L.ba_qkv_project(plan.handle, ctypes.byref(a), stream) == 1, kw  # BA_E_INVALID
    torch.cuda.synchronize()
