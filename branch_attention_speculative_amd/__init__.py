"""Draft branch attention under context parallelism on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/branch_attn.h``: argument
marshalling only. Every step of the computation runs in the HIP kernels of
``libbranch_attn.so``; PyTorch is used for device memory and streams. There
is no fallback: if the library is missing the calls raise.

    plan = Plan(seqlens, cp_degree=8, cp_rank=0, kind=KIND_TTT, depth_or_block=7,
                hq=32, hkv=8, d=128, dtype="bf16")
    plan.upload()
    o, lse, ob, lseb = fwd(plan, q, k, v, qb, kb, vb)
    dq, dk, dv, dqb, dkb, dvb = bwd(plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob)

Tensor layouts are those of the header: q/o [N, hq, d]; k/v [C, N, hkv, d]
(shard s = rank s's local rows); qb/ob [NB, hq, d]; kb/vb [NB, hkv, d];
lse [N, hq], lseb [NB, hq] float32. Element types: dtype "bf16" (bf16
throughout), "fp32" (float32 throughout) or "fp8" (q, k, qb, kb as
torch.float8_e4m3fn, i.e. OCP fp8 E4M3; v, vb, o, ob bf16; the backward
returns bf16 gradients).
"""

import ctypes
import os

import numpy as np

KIND_NONE, KIND_TTT, KIND_BLOCK_BIDIR, KIND_BLOCK_CAUSAL = 0, 1, 2, 3
DTYPES = {"bf16": 0, "fp32": 1, "fp8": 2}

BA_OK = 0
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbranch_attn.so")

_c_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_seqs", "cp_degree", "cp_rank", "kind", "hq", "hkv", "d", "dtype",
                 "max_branch_len", "run_walk")] + \
               [(n, ctypes.c_int64) for n in
                ("n_local_rows", "n_pad_rows", "n_local_anchors", "n_branch_rows",
                 "pairs_main", "pairs_prefix", "pairs_local", "pairs_total")] + \
               [("ws_fwd_bytes", ctypes.c_size_t), ("ws_bwd_bytes", ctypes.c_size_t)]


class Indices(ctypes.Structure):
    _fields_ = [(n, _c_i32p) for n in
                ("cu_real", "cu_pad", "cu_local", "perm", "is_pad", "pos", "seq",
                 "anchor_row", "anchor_pos", "anchor_seq", "branch_off")]


class FwdArgs(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float)] + \
               [(n, ctypes.c_void_p) for n in ("q", "k", "v", "qb", "kb", "vb", "o", "lse",
                                               "ob", "lseb", "workspace")] + \
               [("workspace_bytes", ctypes.c_size_t)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float)] + \
               [(n, ctypes.c_void_p) for n in ("q", "k", "v", "qb", "kb", "vb", "o", "ob",
                                               "lse", "lseb", "dout", "doutb", "dq", "dk", "dv",
                                               "dqb", "dkb", "dvb", "workspace")] + \
               [("workspace_bytes", ctypes.c_size_t)]


class ProjArgs(ctypes.Structure):
    _fields_ = [("target", ctypes.c_int32), ("step", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float)] + \
               [(n, ctypes.c_void_p) for n in ("x", "w", "q_norm", "k_norm", "q", "k", "v")]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class BranchAttnError(RuntimeError):
    pass


_lib = None


def lib():
    """Load ``libbranch_attn.so`` (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        L.ba_plan_create.restype = ctypes.c_int
        L.ba_plan_create.argtypes = [_c_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int, ctypes.c_int32, _c_i32p, ctypes.c_int32, _c_i32p,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_void_p)]
        L.ba_plan_upload.restype = ctypes.c_int
        L.ba_plan_upload.argtypes = [ctypes.c_void_p]
        L.ba_plan_set_walk.restype = ctypes.c_int
        L.ba_plan_set_walk.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.ba_plan_get_info.restype = ctypes.c_int
        L.ba_plan_get_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]
        L.ba_plan_get_indices.restype = ctypes.c_int
        L.ba_plan_get_indices.argtypes = [ctypes.c_void_p, ctypes.POINTER(Indices)]
        L.ba_plan_destroy.restype = None
        L.ba_plan_destroy.argtypes = [ctypes.c_void_p]
        L.branch_attn_fwd.restype = ctypes.c_int
        L.branch_attn_fwd.argtypes = [ctypes.c_void_p, ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.branch_attn_fwd_static.restype = ctypes.c_int
        L.branch_attn_fwd_static.argtypes = [ctypes.c_void_p, ctypes.POINTER(FwdArgs),
                                             ctypes.c_void_p]
        L.branch_attn_bwd.restype = ctypes.c_int
        L.branch_attn_bwd.argtypes = [ctypes.c_void_p, ctypes.POINTER(BwdArgs), ctypes.c_void_p]
        L.ba_plan_get_worklist.restype = ctypes.c_int
        L.ba_plan_get_worklist.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.POINTER(_c_i32p), ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int32)]
        L.ba_qkv_project.restype = ctypes.c_int
        L.ba_qkv_project.argtypes = [ctypes.c_void_p, ctypes.POINTER(ProjArgs), ctypes.c_void_p]
        L.ba_status_str.restype = ctypes.c_char_p
        L.ba_status_str.argtypes = [ctypes.c_int]
        L.ba_last_error.restype = ctypes.c_char_p
        L.ba_last_error.argtypes = []
        L.ba_profile_enable.restype = ctypes.c_int
        L.ba_profile_enable.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.ba_profile_read.restype = ctypes.c_int
        L.ba_profile_read.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32)]
        L.ba_probe_mfma.restype = ctypes.c_int
        L.ba_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
        _lib = L
    return _lib


def _check(status, what):
    if status != BA_OK:
        L = lib()
        raise BranchAttnError(f"{what}: {L.ba_status_str(status).decode()}: "
                              f"{L.ba_last_error().decode()}")


def _i32(arr):
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
    return a, a.ctypes.data_as(_c_i32p)


class Plan:
    """Host plan of one rank (zigzag split, branch index, work lists)."""

    def __init__(self, seqlens, cp_degree, cp_rank, kind, depth_or_block=0, anchors=None,
                 branch_lens=None, hq=32, hkv=8, d=128, dtype="bf16"):
        L = lib()
        self._lens, lp = _i32(seqlens)
        if anchors is not None and len(anchors):
            self._anch, ap = _i32(anchors)
            na = len(self._anch)
        else:
            self._anch, ap, na = None, None, 0
        if branch_lens is not None:
            self._bl, bp = _i32(branch_lens)
        else:
            self._bl, bp = None, None
        self.dtype = dtype
        h = ctypes.c_void_p()
        _check(L.ba_plan_create(lp, len(self._lens), cp_degree, cp_rank, int(kind),
                                int(depth_or_block), ap, na, bp, hq, hkv, d, DTYPES[dtype],
                                ctypes.byref(h)), "ba_plan_create")
        self._h = h
        self.info = self._info()

    def _info(self):
        i = PlanInfo()
        _check(lib().ba_plan_get_info(self._h, ctypes.byref(i)), "ba_plan_get_info")
        return {n: getattr(i, n) for n, _ in PlanInfo._fields_}

    def indices(self):
        """Host copies of the plan's index arrays (numpy int32)."""
        x = Indices()
        _check(lib().ba_plan_get_indices(self._h, ctypes.byref(x)), "ba_plan_get_indices")
        S = self.info["n_seqs"]
        N = self.info["n_local_rows"]
        A = self.info["n_local_anchors"]
        sizes = dict(cu_real=S + 1, cu_pad=S + 1, cu_local=S + 1, perm=N, is_pad=N, pos=N, seq=N,
                     anchor_row=A, anchor_pos=A, anchor_seq=A, branch_off=A + 1)
        out = {}
        for name, n in sizes.items():
            ptr = getattr(x, name)
            out[name] = np.ctypeslib.as_array(ptr, shape=(n,)).copy() if n else np.zeros(0, np.int32)
        return out

    def worklist(self, which):
        """Host copy of a kernel work list as an int32 array [tiles, ints per tile]
        (0: query tiles, 1: key tiles, 2: branch tiles)."""
        ptr = _c_i32p()
        n = ctypes.c_int64()
        w = ctypes.c_int32()
        _check(lib().ba_plan_get_worklist(self._h, int(which), ctypes.byref(ptr), ctypes.byref(n),
                                          ctypes.byref(w)), "ba_plan_get_worklist")
        if n.value == 0:
            return np.zeros((0, w.value), np.int32)
        return np.ctypeslib.as_array(ptr, shape=(n.value * w.value,)).reshape(n.value, w.value).copy()

    def set_walk(self, mode):
        """Key walk of the forward and dQ kernels: "auto", "segments" or "runs"."""
        _check(lib().ba_plan_set_walk(self._h, {"auto": 0, "segments": 1, "runs": 2}[mode]),
               "ba_plan_set_walk")
        self.info = self._info()
        return self

    def upload(self):
        """Copy index arrays and work lists to the current HIP device."""
        _check(lib().ba_plan_upload(self._h), "ba_plan_upload")
        return self

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().ba_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# device calls (torch for memory and streams)


def _torch():
    import torch
    return torch


def _tdtype(plan):
    """Element type of v, vb, o, ob and of the gradients."""
    t = _torch()
    return t.float32 if plan.dtype == "fp32" else t.bfloat16


def _qkdtype(plan):
    """Element type of q, k, qb, kb."""
    t = _torch()
    return t.float8_e4m3fn if plan.dtype == "fp8" else _tdtype(plan)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(ws, need, device):
    """Byte size of a caller-supplied workspace after checking that it is a
    contiguous tensor on the right device (its dtype does not matter)."""
    if ws.device != device:
        raise ValueError(f"workspace: expected device {device}, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace: needs {need} bytes, got {nbytes}")
    return nbytes


def _shapes(plan):
    i = plan.info
    N, NB, C = i["n_local_rows"], i["n_branch_rows"], i["cp_degree"]
    hq, hkv, d = i["hq"], i["hkv"], i["d"]
    return dict(q=(N, hq, d), k=(C, N, hkv, d), qb=(NB, hq, d), kb=(NB, hkv, d),
                lse=(N, hq), lseb=(NB, hq))


def fwd(plan, q, k, v, qb=None, kb=None, vb=None, scale=0.0, workspace=None):
    """Forward; returns (o, lse, ob, lseb). ``scale <= 0`` means 1/sqrt(d)."""
    torch = _torch()
    dev = q.device
    dt = _tdtype(plan)
    dq8 = _qkdtype(plan)
    S = _shapes(plan)
    nb = plan.info["n_branch_rows"]
    _expect("q", q, S["q"], dq8, dev)
    _expect("k", k, S["k"], dq8, dev)
    _expect("v", v, S["k"], dt, dev)
    if nb:
        _expect("qb", qb, S["qb"], dq8, dev)
        _expect("kb", kb, S["kb"], dq8, dev)
        _expect("vb", vb, S["kb"], dt, dev)
    o = torch.empty(S["q"], dtype=dt, device=dev)
    lse = torch.empty(S["lse"], dtype=torch.float32, device=dev)
    ob = torch.empty(S["qb"], dtype=dt, device=dev) if nb else None
    lseb = torch.empty(S["lseb"], dtype=torch.float32, device=dev) if nb else None
    ws_bytes = plan.info["ws_fwd_bytes"]
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    a = FwdArgs(scale=float(scale), q=_ptr(q), k=_ptr(k), v=_ptr(v), qb=_ptr(qb), kb=_ptr(kb),
                vb=_ptr(vb), o=_ptr(o), lse=_ptr(lse), ob=_ptr(ob), lseb=_ptr(lseb),
                workspace=_ptr(workspace),
                workspace_bytes=0 if workspace is None else _workspace(workspace, ws_bytes, dev))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(lib().branch_attn_fwd(plan.handle, ctypes.byref(a), ctypes.c_void_p(stream)),
               "branch_attn_fwd")
    return o, lse, ob, lseb


def fwd_static(plan, q, k, v, qb=None, kb=None, vb=None, out=None, scale=0.0):
    """Forward through ``branch_attn_fwd_static``: no workspace, so nothing is
    allocated when the outputs are given as ``out = (o, lse, ob, lseb)``
    (ob/lseb None without branch rows); otherwise they are allocated here.
    Returns (o, lse, ob, lseb)."""
    torch = _torch()
    dev = q.device
    dt = _tdtype(plan)
    dq8 = _qkdtype(plan)
    S = _shapes(plan)
    nb = plan.info["n_branch_rows"]
    _expect("q", q, S["q"], dq8, dev)
    _expect("k", k, S["k"], dq8, dev)
    _expect("v", v, S["k"], dt, dev)
    if nb:
        _expect("qb", qb, S["qb"], dq8, dev)
        _expect("kb", kb, S["kb"], dq8, dev)
        _expect("vb", vb, S["kb"], dt, dev)
    if out is None:
        out = (torch.empty(S["q"], dtype=dt, device=dev),
               torch.empty(S["lse"], dtype=torch.float32, device=dev),
               torch.empty(S["qb"], dtype=dt, device=dev) if nb else None,
               torch.empty(S["lseb"], dtype=torch.float32, device=dev) if nb else None)
    o, lse, ob, lseb = out
    _expect("o", o, S["q"], dt, dev)
    _expect("lse", lse, S["lse"], torch.float32, dev)
    if nb:
        _expect("ob", ob, S["qb"], dt, dev)
        _expect("lseb", lseb, S["lseb"], torch.float32, dev)
    a = FwdArgs(scale=float(scale), q=_ptr(q), k=_ptr(k), v=_ptr(v), qb=_ptr(qb), kb=_ptr(kb),
                vb=_ptr(vb), o=_ptr(o), lse=_ptr(lse), ob=_ptr(ob), lseb=_ptr(lseb),
                workspace=None, workspace_bytes=0)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(lib().branch_attn_fwd_static(plan.handle, ctypes.byref(a), ctypes.c_void_p(stream)),
               "branch_attn_fwd_static")
    return o, lse, ob, lseb


def bwd(plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob, scale=0.0, workspace=None):
    """Backward; returns (dq, dk, dv, dqb, dkb, dvb). For fp8 plans the
    gradients are bf16."""
    torch = _torch()
    dev = q.device
    dt, qt = _tdtype(plan), _qkdtype(plan)
    S = _shapes(plan)
    nb = plan.info["n_branch_rows"]
    for name, t, shp, ty in (("q", q, S["q"], qt), ("k", k, S["k"], qt), ("v", v, S["k"], dt),
                             ("o", o, S["q"], dt), ("do", do, S["q"], dt)):
        _expect(name, t, shp, ty, dev)
    _expect("lse", lse, S["lse"], torch.float32, dev)
    if nb:
        for name, t, shp, ty in (("qb", qb, S["qb"], qt), ("kb", kb, S["kb"], qt),
                                 ("vb", vb, S["kb"], dt), ("ob", ob, S["qb"], dt),
                                 ("dob", dob, S["qb"], dt)):
            _expect(name, t, shp, ty, dev)
        _expect("lseb", lseb, S["lseb"], torch.float32, dev)
    dq = torch.empty(S["q"], dtype=dt, device=dev)
    dk = torch.empty(S["k"], dtype=dt, device=dev)
    dv = torch.empty(S["k"], dtype=dt, device=dev)
    dqb = torch.empty(S["qb"], dtype=dt, device=dev) if nb else None
    dkb = torch.empty(S["kb"], dtype=dt, device=dev) if nb else None
    dvb = torch.empty(S["kb"], dtype=dt, device=dev) if nb else None
    if workspace is None:
        workspace = torch.empty(plan.info["ws_bwd_bytes"], dtype=torch.uint8, device=dev)
    a = BwdArgs(scale=float(scale), q=_ptr(q), k=_ptr(k), v=_ptr(v), qb=_ptr(qb), kb=_ptr(kb),
                vb=_ptr(vb), o=_ptr(o), ob=_ptr(ob), lse=_ptr(lse), lseb=_ptr(lseb),
                dout=_ptr(do), doutb=_ptr(dob), dq=_ptr(dq), dk=_ptr(dk), dv=_ptr(dv),
                dqb=_ptr(dqb), dkb=_ptr(dkb), dvb=_ptr(dvb), workspace=_ptr(workspace),
                workspace_bytes=_workspace(workspace, plan.info["ws_bwd_bytes"], dev))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(lib().branch_attn_bwd(plan.handle, ctypes.byref(a), ctypes.c_void_p(stream)),
               "branch_attn_bwd")
    return dq, dk, dv, dqb, dkb, dvb


def qkv_project(plan, x, w, q_norm=None, k_norm=None, branch=False, step=-1, rope_theta=1e6,
                eps=1e-6, out=None):
    """Draft-layer projection (``ba_qkv_project``): q, k, v of the rows of
    hidden states ``x`` [rows, hidden] with ``w`` [(hq + 2 hkv) d, hidden],
    per-head RMS norm of q and k when ``q_norm``/``k_norm`` [d] are given, and
    RoPE at each row's position (``rope_theta <= 0``: none). Main rows
    (branch=False) give q [N, hq, d], k, v [N, hkv, d]; branch rows give
    qb [NB, hq, d], kb, vb [NB, hkv, d]; ``step = j`` takes one row per local
    anchor (a TTT pass) and fills branch row j of every anchor in ``out``
    (required then). Returns (q, k, v)."""
    torch = _torch()
    dev = x.device
    i = plan.info
    hq, hkv, d = i["hq"], i["hkv"], i["d"]
    hidden = x.shape[1]
    rows = i["n_branch_rows"] if branch else i["n_local_rows"]
    if step >= 0:
        if out is None:
            raise ValueError("a TTT step pass fills given qb/kb/vb tensors: pass out=(qb, kb, vb)")
        _expect("x", x, (i["n_local_anchors"], hidden), torch.bfloat16, dev)
    else:
        _expect("x", x, (rows, hidden), torch.bfloat16, dev)
    _expect("w", w, ((hq + 2 * hkv) * d, hidden), torch.bfloat16, dev)
    for name, t in (("q_norm", q_norm), ("k_norm", k_norm)):
        if t is not None:
            _expect(name, t, (d,), torch.bfloat16, dev)
    if out is None:
        out = (torch.empty((rows, hq, d), dtype=torch.bfloat16, device=dev),
               torch.empty((rows, hkv, d), dtype=torch.bfloat16, device=dev),
               torch.empty((rows, hkv, d), dtype=torch.bfloat16, device=dev))
    q, k, v = out
    _expect("q", q, (rows, hq, d), torch.bfloat16, dev)
    _expect("k", k, (rows, hkv, d), torch.bfloat16, dev)
    _expect("v", v, (rows, hkv, d), torch.bfloat16, dev)
    a = ProjArgs(target=1 if branch else 0, step=int(step), hidden=int(hidden),
                 rope_theta=float(rope_theta), norm_eps=float(eps), x=_ptr(x), w=_ptr(w),
                 q_norm=_ptr(q_norm), k_norm=_ptr(k_norm), q=_ptr(q), k=_ptr(k), v=_ptr(v))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(lib().ba_qkv_project(plan.handle, ctypes.byref(a), ctypes.c_void_p(stream)),
               "ba_qkv_project")
    return q, k, v


def profile_enable(on=True, max_launches=4096):
    """Bracket every kernel launch with HIP events on its stream."""
    _check(lib().ba_profile_enable(1 if on else 0, int(max_launches)), "ba_profile_enable")


def profile_read():
    """{kernel name: (launches, total_ms)} since the last read; synchronises."""
    n = ctypes.c_int32(0)
    buf = (KernelTime * 64)()
    _check(lib().ba_profile_read(buf, 64, ctypes.byref(n)), "ba_profile_read")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n.value, 64))}


def _autograd():
    torch = _torch()

    class BranchAttnFunction(torch.autograd.Function):
        """torch.autograd wrapper: forward = branch_attn_fwd, backward =
        branch_attn_bwd. Returns (o, ob)."""

        @staticmethod
        def forward(ctx, plan, scale, q, k, v, qb, kb, vb):
            o, lse, ob, lseb = fwd(plan, q, k, v, qb, kb, vb, scale=scale)
            ctx.plan, ctx.scale = plan, scale
            ctx.save_for_backward(q, k, v, qb, kb, vb, o, lse, ob, lseb)
            return o, ob

        @staticmethod
        def backward(ctx, do, dob):
            q, k, v, qb, kb, vb, o, lse, ob, lseb = ctx.saved_tensors
            do = do.contiguous()
            dob = dob.contiguous() if dob is not None else None
            g = bwd(ctx.plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob, scale=ctx.scale)
            return (None, None) + tuple(g)

    return BranchAttnFunction


def branch_attention(plan, q, k, v, qb=None, kb=None, vb=None, scale=0.0):
    """Differentiable branch attention (torch.autograd); returns (o, ob)."""
    return _autograd().apply(plan, scale, q, k, v, qb, kb, vb)


def probe_mfma(random_operands=True, iters=20000, device=None):
    """Dense bf16 MFMA rate (TFLOP/s) that the part sustains on register
    operands: all zero, or pseudo-random values that change every MFMA.
    Synchronises. A measurement aid, not part of the attention path."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    sink = torch.empty(8192, dtype=torch.float32, device=dev)
    out = ctypes.c_double(0.0)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(lib().ba_probe_mfma(1 if random_operands else 0, int(iters), ctypes.c_void_p(sink.data_ptr()),
                                   sink.numel(), ctypes.c_void_p(stream), ctypes.byref(out)),
               "ba_probe_mfma")
    return out.value
