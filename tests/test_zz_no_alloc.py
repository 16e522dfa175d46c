"""The no-allocation forward (branch_attn_fwd_static) through the C ABI: the
same outputs as branch_attn_fwd with a caller workspace, on two calls in a
row, the second on a plan with a smaller workspace, so the static scratch
holds the first call's data when the second starts; and plans whose
workspace exceeds the scratch are rejected before anything is read."""

import ctypes

import pytest

import workloads

from helpers import inputs, make_plan, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import branch_attention_speculative_amd as ba
    ba.lib()
    return torch, ba


def _fwd_args(ba, dev, out, workspace=None, ws_bytes=0):
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    o, lse, ob, lseb = out
    return ba.FwdArgs(scale=0.0, q=p(dev["q"]), k=p(dev["k"]), v=p(dev["v"]), qb=p(dev["qb"]),
                      kb=p(dev["kb"]), vb=p(dev["vb"]), o=p(o), lse=p(lse), ob=p(ob),
                      lseb=p(lseb), workspace=p(workspace), workspace_bytes=ws_bytes)


def _outputs(torch, plan):
    i = plan.info
    N, NB, hq, d = i["n_local_rows"], i["n_branch_rows"], i["hq"], i["d"]
    dt = torch.bfloat16 if plan.dtype == "bf16" else torch.float32
    mk = lambda shp, t: torch.full(shp, 7.0, dtype=t, device="cuda")
    return (mk((N, hq, d), dt), mk((N, hq), torch.float32),
            mk((NB, hq, d), dt) if NB else None, mk((NB, hq), torch.float32) if NB else None)


def test_static_forward_equals_the_workspace_forward_on_two_calls_in_a_row(env):
    torch, ba = env
    L = ba.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sizes = []
    for name in ("long256k_r", "dflash_r"):  # the second plan's workspace is the smaller
        w = workloads.make(name)
        plan = make_plan(ba, w)
        ws_bytes = plan.info["ws_fwd_bytes"]
        sizes.append(ws_bytes)
        say(f"[case] static forward, {name}: workspace {ws_bytes} bytes")
        raw, _ = inputs(w, plan.info["n_local_rows"], plan.info["n_branch_rows"],
                        names=["q", "k", "v", "qb", "kb", "vb"])
        dev = {k: to_device(torch, w, v) for k, v in raw.items()}
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        ref = _outputs(torch, plan)
        assert L.branch_attn_fwd(plan.handle, ctypes.byref(_fwd_args(ba, dev, ref, ws, ws_bytes)),
                                 stream) == 0
        got = _outputs(torch, plan)
        assert L.branch_attn_fwd_static(plan.handle, ctypes.byref(_fwd_args(ba, dev, got)),
                                        stream) == 0, L.ba_last_error()
        torch.cuda.synchronize()
        for x, y, nm in zip(got, ref, ("o", "lse", "ob", "lseb")):
            if y is not None:
                assert torch.equal(x, y), (name, nm)
        say("  static forward bit-identical to the workspace forward")
    assert sizes[1] < sizes[0]


def test_static_forward_rejects_plans_beyond_the_scratch(env):
    torch, ba = env
    L = ba.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    w = workloads.make("long256k")  # 3.7 GB forward workspace
    plan = make_plan(ba, w)
    assert plan.info["ws_fwd_bytes"] > (256 << 20)
    # no tensors at all: the size check comes before any argument is read,
    # and NULL inputs could never be launched on
    args = ba.FwdArgs(scale=0.0)
    assert L.branch_attn_fwd_static(plan.handle, ctypes.byref(args), stream) == 3  # BA_E_WORKSPACE
    assert b"static scratch" in L.ba_last_error()
    # a caller workspace is refused as well
    small = workloads.make("dflash_r")
    sp = make_plan(ba, small)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    args = ba.FwdArgs(scale=0.0, workspace=ctypes.c_void_p(ws.data_ptr()), workspace_bytes=16)
    assert L.branch_attn_fwd_static(sp.handle, ctypes.byref(args), stream) == 1  # BA_E_INVALID
    torch.cuda.synchronize()
