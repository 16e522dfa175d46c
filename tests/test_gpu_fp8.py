"""GPU parity of the fp8 path (dtype "fp8": Q, K, Qb, Kb as OCP fp8 E4M3
codes, V, Vb, O, Ob bf16) through the C ABI, against the oracle fed the same
decoded fp8 values. The pages name fp8 as a precision to watch for the
online-softmax merge (rainbus analysis, weaknesses and improvements, item 4);
the tolerances are the bf16 ones: O max-abs <= 2e-2 and rel-L2 <= 1e-2, LSE
max-abs <= 1e-3, gradients as for bf16 inputs. The backward takes the E4M3
values as bf16 and runs the bf16 backward, except that the dQ kernel forms
the scores on the fp8 matrix cores; one test checks it against the bf16 plan
on the decoded values: dK, dV, dKb, dVb bit for bit, dQ and dQb to a
rounding-order bound. The inputs are the bf16 workloads' seeded N(0, 1)
draws, encoded to E4M3 for the score operands."""


import numpy as np
import pytest

import workloads
from oracle import pack

from helpers import LazyF32, grad_ok, inputs, lse_err, make_plan, max_abs, oracle_grouped, \
    oracle_structs, random_workload, rel_l2, say, subset_grouped, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import branch_attention_speculative_amd as ba
    ba.lib()
    return torch, ba


def _fp8(w):
    return workloads.Workload(w.name + "-fp8", w.seqlens, w.C, w.r, w.kind, w.depth_or_block, w.hq,
                              w.hkv, w.d, "fp8", False, w.seed, anchors=w.anchors,
                              branch_lens=w.branch_lens)


def _check(name, go, wo, gl, wl):
    e_o, r_o, e_l = max_abs(go, wo), rel_l2(go, wo), lse_err(gl, wl)
    say(f"  {name}: max|dO|={e_o:.3e} relL2={r_o:.3e} max|dLSE|={e_l:.3e}")
    assert e_o <= 2e-2 and r_o <= 1e-2 and e_l <= 1e-3, (name, e_o, r_o, e_l)


def _run(env, w):
    torch, ba = env
    say(f"[case] fp8 {w.name}: lens={w.seqlens[:6]} C={w.C} r={w.r} kind={w.kind} "
        f"heads={w.hq}/{w.hkv}")
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    N, NB = plan.info["n_local_rows"], plan.info["n_branch_rows"]
    raw, dec = inputs(w, N, NB, names=["q", "k", "v", "qb", "kb", "vb"])
    assert raw["q"].dtype == np.uint8 and raw["v"].dtype == np.uint16
    dev = {k: to_device(torch, w, v) for k, v in raw.items()}
    o, lse, ob, lseb = ba.fwd(plan, dev["q"], dev["k"], dev["v"], dev["qb"], dev["kb"], dev["vb"])
    torch.cuda.synchronize()
    ref = oracle_grouped(lay, br, *(dec[k] for k in ("q", "k", "v", "qb", "kb", "vb")))
    _check("o", to_host(o), ref["o"], to_host(lse), ref["lse"])
    if NB:
        _check("ob", to_host(ob), ref["ob"], to_host(lseb), ref["lseb"])
    return plan, dev


@pytest.mark.parametrize("name", ["ttt32k_r", "dflash_r", "long256k_r", "dspark_r"])
def test_fp8_forward_reduced_workloads(env, name):
    _run(env, _fp8(workloads.make(name)))


def _edge(name, lens, C, r, kind, depth, hq, hkv, anchors=None, blens=None):
    seed = sum(ord(ch) for ch in name)
    return workloads.Workload(name, lens, C, r, kind, depth, hq, hkv, 128, "fp8", False, seed,
                              anchors=anchors, branch_lens=blens)


@pytest.mark.parametrize("w", [
    # plain causal ring attention, C=1, one-token and odd-length sequences
    _edge("fp8-none-c1", [1, 2, 3, 130], 1, 0, pack.KIND_NONE, 0, 4, 2),
    # sequences shorter than 2C (pad rows), a long ragged chunk, G=16
    _edge("fp8-short-c8", [5, 3, 17, 1], 8, 5, pack.KIND_TTT, 2, 8, 2),
    _edge("fp8-ragged", [1999], 3, 1, pack.KIND_TTT, 2, 8, 2),
    _edge("fp8-g16", [257, 100], 4, 2, pack.KIND_BLOCK_CAUSAL, 0, 16, 1,
          anchors=[3, 100, 256, 300], blens=[8, 16, 8, 16]),
    # blocks of 1 and of 64 keys, bidirectional
    _edge("fp8-block-edges", [40, 200], 2, 1, pack.KIND_BLOCK_BIDIR, 0, 16, 4,
          anchors=[0, 39, 40, 150, 239], blens=[1, 64, 5, 64, 1]),
], ids=lambda w: w.name)
def test_fp8_forward_edge_cases(env, w):
    _run(env, w)


def test_fp8_forward_full_size_long256k_sampled(env):
    """The 262,144-token share in fp8: the first and last 64 rows of both local
    chunks with all their TTT branch rows, against the oracle's dense form of
    that row subset."""
    torch, ba = env
    w = _fp8(workloads.make("long256k"))
    say("[case] fp8 full-size long256k")
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    N, NB = plan.info["n_local_rows"], plan.info["n_branch_rows"]
    raw = workloads.draw(w, N, NB, names=["q", "k", "v", "qb", "kb", "vb"])
    dev = {k: to_device(torch, w, v) for k, v in raw.items()}
    o, lse, ob, lseb = ba.fwd(plan, dev["q"], dev["k"], dev["v"], dev["qb"], dev["kb"], dev["vb"])
    torch.cuda.synchronize()
    c = int(lay["c"][0])
    e = 64
    rows = np.array(sorted(set(range(e)) | set(range(c - e, c)) | set(range(c, c + e)) |
                           set(range(2 * c - e, 2 * c))), np.int64)
    anch = np.nonzero(np.isin(br["anchor_row"], rows))[0]
    L = {k: LazyF32(w, v) for k, v in raw.items()}
    ref = subset_grouped(lay, br, L["q"], L["k"], L["v"], L["qb"], L["kb"], L["vb"], rows, anch)
    brows = ref["branch_rows"]
    ri = torch.tensor(rows, device="cuda")
    bi = torch.tensor(brows, device="cuda", dtype=torch.long)
    _check("o", to_host(o[ri]), ref["o"], to_host(lse[ri]), ref["lse"])
    _check("ob", to_host(ob[bi]), ref["ob"], to_host(lseb[bi]), ref["lseb"])


@pytest.mark.parametrize("name", ["ttt32k_r", "dflash_r", "dspark_r"])
def test_fp8_backward_matches_the_oracle(env, name):
    """Forward and backward on an fp8 plan against the oracle's dense
    backward on the decoded values (the gradients are bf16)."""
    _fwd_bwd_against_oracle(env, _fp8(workloads.make(name)))


FP8_RANDOM = [random_workload(i, "fp8") for i in range(32)]


@pytest.mark.parametrize("w", FP8_RANDOM, ids=[w.name for w in FP8_RANDOM])
def test_fp8_random_configurations(env, w):
    """Seeded random shapes (every branch kind, C up to 16, GQA groups up to
    16): the fp8 forward and backward against the oracle."""
    _fwd_bwd_against_oracle(env, w)


def _fwd_bwd_against_oracle(env, w):
    torch, ba = env
    say(f"[case] fp8 fwd+bwd {w.name}: lens={w.seqlens[:6]} C={w.C} r={w.r} kind={w.kind} "
        f"heads={w.hq}/{w.hkv}")
    lay, br = oracle_structs(w)
    plan = make_plan(ba, w)
    N, NB = plan.info["n_local_rows"], plan.info["n_branch_rows"]
    raw, dec = inputs(w, N, NB)
    dev = {k: to_device(torch, w, v) for k, v in raw.items()}
    o, lse, ob, lseb = ba.fwd(plan, dev["q"], dev["k"], dev["v"], dev["qb"], dev["kb"], dev["vb"])
    g = ba.bwd(plan, dev["q"], dev["k"], dev["v"], dev["qb"], dev["kb"], dev["vb"], o, lse, ob, lseb,
               dev["do"], dev["dob"])
    torch.cuda.synchronize()
    assert all(t is None or t.dtype == torch.bfloat16 for t in g)
    ref = oracle_grouped(lay, br, *(dec[k] for k in ("q", "k", "v", "qb", "kb", "vb")), dec["do"],
                         dec["dob"])
    _check("o", to_host(o), ref["o"], to_host(lse), ref["lse"])
    if NB:
        _check("ob", to_host(ob), ref["ob"], to_host(lseb), ref["lseb"])
    for nm, t in zip(("dq", "dk", "dv", "dqb", "dkb", "dvb"), g):
        got = to_host(t) if t is not None else np.zeros(0)
        ok, ma, rl = grad_ok(got, ref[nm], True)
        say(f"  {nm}: max-abs={ma:.3e} relL2={rl:.3e}")
        assert ok, (nm, ma, rl)


def test_fp8_backward_equals_the_bf16_backward_on_decoded_values(env):
    """Every E4M3 value is a bf16 value: the fp8 plan's backward and the bf16
    plan's backward on q, k, qb, kb decoded to bf16 (same O, LSE and dO) give
    identical dK, dV, dKb, dVb. dQ and dQb differ only in the fp32 rounding
    order of the scores in the dQ kernel (fp8 products summed 64 at a time
    against 16). That moves P by a few fp32 steps, which can move a dS
    element across a bf16 rounding boundary before the dS K product, so
    single dQ elements may move by a few bf16 steps of their larger terms.
    The bound: the bf16 gradient one (max-abs <= 2e-2 * max(1, |dQ|_inf)) and
    relative L2 <= 2e-3 (about 4e-4 measured on this workload)."""
    torch, ba = env
    w8 = _fp8(workloads.make("long256k_r"))
    w16 = workloads.make("long256k_r")
    p8, p16 = make_plan(ba, w8), make_plan(ba, w16)
    N, NB = p8.info["n_local_rows"], p8.info["n_branch_rows"]
    raw, _ = inputs(w8, N, NB)
    dev = {k: to_device(torch, w8, v) for k, v in raw.items()}
    o, lse, ob, lseb = ba.fwd(p8, dev["q"], dev["k"], dev["v"], dev["qb"], dev["kb"], dev["vb"])
    as16 = {k: dev[k].to(torch.bfloat16) for k in ("q", "k", "qb", "kb")}
    g8 = ba.bwd(p8, dev["q"], dev["k"], dev["v"], dev["qb"], dev["kb"], dev["vb"], o, lse, ob, lseb,
                dev["do"], dev["dob"])
    g16 = ba.bwd(p16, as16["q"], as16["k"], dev["v"], as16["qb"], as16["kb"], dev["vb"], o, lse, ob,
                 lseb, dev["do"], dev["dob"])
    torch.cuda.synchronize()
    for nm, a, b in zip(("dq", "dk", "dv", "dqb", "dkb", "dvb"), g8, g16):
        if nm in ("dq", "dqb"):
            a, b = to_host(a).astype(np.float64), to_host(b).astype(np.float64)
            d = np.abs(a - b)
            rl = rel_l2(a, b)
            say(f"  {nm}: {np.count_nonzero(d)} of {d.size} differ, max {d.max():.3e}, "
                f"relL2 {rl:.3e}")
            assert rl <= 2e-3 and d.max() <= 2e-2 * max(1.0, np.max(np.abs(b))), (nm, rl, d.max())
        else:
            assert torch.equal(a, b), nm
    say(f"  fp8 and bf16 backward agree on {N} rows + {NB} branch rows")
