#!/usr/bin/env python3
"""Benchmark: draft branch attention fwd+bwd on one MI355X.

One step = one full pass of the hot path over one synthetic batch: the
forward (ring-step causal partial over every virtual ring step, branch-local
partial, Eq. 2 merge) and the backward (Delta, branch-local backward, dQ and
dK/dV ring replay). Inputs are resident in device memory before timing.

Throughput is effective TFLOP/s over unmasked (query row, key) pairs only:
4*D FLOP per pair per q-head forward (Q K^T and P V), 10*D backward
(recomputed Q K^T, dO V^T, dV, dQ, dK). Pads are excluded.

Prints one JSON line. Default workload: one 262,144-token sequence at virtual
CP=8, rank 0's share (32,768 local rows, 229,376 EAGLE-3 TTT branch rows of
depth 7), 32 q-heads / 8 kv-heads, d=128, bf16.
"""

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096)
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 matrix-core peak (256 CU x 2.4 GHz x 8192)
# the fp8 forward does half its FLOPs (Q K^T) at the fp8 rate, half (P V) at the bf16 rate
PEAK_FP8_QK_BF16_PV_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0
METRIC = "branch-attn fwd+bwd effective TFLOP/s (1 GPU) and % of bf16 MFMA peak"
METRIC_FP8 = ("branch-attn fwd effective TFLOP/s (1 GPU), fp8 E4M3 Q K^T with bf16 P V, and % of "
              "the matching fp8/bf16 MFMA peak")
METRIC_FP8_STEP = ("branch-attn fwd+bwd effective TFLOP/s (1 GPU), fp8 E4M3 Q/K scores with bf16 "
                   "elsewhere, and % of the matching fp8/bf16 MFMA peak")
# the fp8 fwd+bwd step is credited 14 D per pair, of which the forward's Q K^T
# and the backward's Q K^T recompute (4 D) are counted at the fp8 rate and the
# other ten at the bf16 rate (the dQ kernel forms its scores in fp8, dK/dV in
# bf16: counting both at the fp8 rate gives the higher, stricter peak)
PEAK_FP8_STEP_TFLOPS = 14.0 / (4.0 / PEAK_FP8_TFLOPS + 10.0 / PEAK_BF16_TFLOPS)

# algorithmic FLOP per unmasked pair per q-head and per unit of D, per kernel:
# the forward ring kernel does Q K^T and P V over the main keys; the dK/dV
# kernel does the four backward contractions over the main keys (Q K^T
# recompute, dO V^T, P^T dO, dS^T Q); the dQ kernel is credited only dS K
# (its Q K^T and dO V^T recomputes are not counted).
KERNEL_FLOP_PER_PAIR_D = {"fwd_ring": 4, "bwd_dkdv": 8, "bwd_dq": 2}
KERNEL_SOURCES = {"fwd_ring": ["fwd_ring.hip", "ring_common.h", "common.h"],
                  "bwd_dkdv": ["bwd_ring.hip", "ring_common.h", "common.h"],
                  "bwd_dq": ["bwd_ring.hip", "ring_common.h", "common.h"]}


def describe(w, info):
    kind = {0: "no branches", 1: f"EAGLE-3 TTT depth {w.depth_or_block}",
            2: "DFlash bidirectional blocks", 3: "DSpark causal blocks"}[w.kind]
    dt = "fp8 E4M3 q/k, bf16 v/o" if w.dtype == "fp8" else w.dtype
    passes = "fwd+bwd" if w.bwd else "fwd"
    return (f"{w.name}: {len(w.seqlens)} seq / {sum(w.seqlens)} tokens, virtual CP={w.C} rank {w.r} "
            f"share ({info['n_local_rows']} local rows, {info['n_branch_rows']} branch rows), "
            f"{w.hq}/{w.hkv} heads, d={w.d}, {dt}, {kind}, {passes}")


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "branch_attention_speculative_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, used
    only if the kernel sources still hash to the value recorded there."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    m_h = re.search(r"source_hash:\s*([0-9a-f]+)", txt)
    if not (m_b and m_h) or m_h.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return float(m_b.group(1))


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, plan_info, raw, n_anchor_sample, seed=11):
    """The oracle, as it stands, on a bounded sample of the same workload:
    the main row and every branch row of ``n_anchor_sample`` seeded anchors,
    forward and backward (their dQ and their dK/dV contributions), against
    their full visible key sets."""
    from threadpoolctl import threadpool_info
    from oracle import attn, pack

    class Lazy:
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def __getitem__(self, idx):
            return workloads.as_f32(w, self.a[idx])

    lay = pack.zigzag_layout(w.seqlens, w.C, w.r)
    if w.kind == pack.KIND_TTT:
        br = pack.branch_index(lay, w.kind, w.depth_or_block)
    elif w.kind == pack.KIND_NONE:
        br = pack.branch_index(lay, w.kind)
    else:
        br = pack.branch_index(lay, w.kind, w.depth_or_block, w.anchors, w.branch_lens)
    rng = np.random.default_rng(seed)
    A = br["anchor_row"].size
    pick = np.sort(rng.choice(A, size=min(n_anchor_sample, A), replace=False))
    main_rows = br["anchor_row"][pick].tolist()
    branch_rows = [b for a in pick for b in range(br["branch_off"][a], br["branch_off"][a + 1])]
    L = {k: Lazy(v) for k, v in raw.items()}
    dk_acc, dv_acc = {}, {}
    t0 = time.perf_counter()
    if w.bwd:
        attn.attn_rows(lay, br, L["q"], L["k"], L["v"], L["qb"], L["kb"], L["vb"], main_rows,
                       branch_rows, dtype=np.float32, do=L["do"], dob=L["dob"], dk_acc=dk_acc,
                       dv_acc=dv_acc)
    else:
        attn.attn_rows(lay, br, L["q"], L["k"], L["v"], L["qb"], L["kb"], L["vb"], main_rows,
                       branch_rows, dtype=np.float32)
    dt = time.perf_counter() - t0
    # unmasked pairs of the sampled rows, from the visibility rules
    pairs = int(np.sum(lay["pos"][main_rows] + 1))
    for b in branch_rows:
        a = br["b_anchor"][b]
        n = br["branch_off"][a + 1] - br["branch_off"][a]
        own = n if br["kind"] == pack.KIND_BLOCK_BIDIR else br["b_j"][b] + 1
        pairs += int(br["anchor_pos"][a]) + 1 + int(own)
    flop = pairs * w.hq * w.d * (14 if w.bwd else 4)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    total_pairs = plan_info["pairs_total"]
    return {
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{len(main_rows)} anchors of the same workload: their {len(main_rows)} main rows "
                   f"+ {len(branch_rows)} branch rows x {w.hq} heads, "
                   f"{'fwd+bwd' if w.bwd else 'fwd'} against full key sets "
                   f"({pairs} of {total_pairs} pairs per head, {dt:.1f} s, fp32 NumPy)"),
        "seconds": dt, "extrapolated_step_s": dt * total_pairs / max(pairs, 1),
    }


def bench_proj(args, ba, torch, w, plan):
    """The draft-layer projection of every main and branch row of the
    workload: q, k, v = x W^T with per-head RMS norm and RoPE, bf16, at
    model width --hidden. One step = both calls."""
    info = plan.info
    N, NB, hid = info["n_local_rows"], info["n_branch_rows"], args.hidden
    nout = (w.hq + 2 * w.hkv) * w.d
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    xm = torch.randn((N, hid), generator=gen, device="cuda").to(torch.bfloat16)
    xb = torch.randn((NB, hid), generator=gen, device="cuda").to(torch.bfloat16)
    W = (torch.randn((nout, hid), generator=gen, device="cuda") / hid ** 0.5).to(torch.bfloat16)
    qn = torch.ones(w.d, dtype=torch.bfloat16, device="cuda")
    kn = torch.ones(w.d, dtype=torch.bfloat16, device="cuda")
    om = ba.qkv_project(plan, xm, W, qn, kn)
    ob = ba.qkv_project(plan, xb, W, qn, kn, branch=True)

    def step():
        ba.qkv_project(plan, xm, W, qn, kn, out=om)
        ba.qkv_project(plan, xb, W, qn, kn, branch=True, out=ob)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ba.profile_enable(True, max_launches=4 * args.steps + 8)
    ba.profile_read()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kern = ba.profile_read()
    ba.profile_enable(False)
    flop = 2.0 * (N + NB) * hid * nout
    n, tot = kern.get("qkv_project", (0, 0.0))
    kms = tot / args.steps
    byt = 2.0 * ((N + NB) * hid + nout * hid + (N + NB) * nout)
    out = {"metric": "draft-layer Q/K/V projection + RMS norm + RoPE, TFLOP/s (1 GPU) and % of bf16 "
                     "MFMA peak", "value": flop / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (random bf16 hidden states and weights)",
           "config": {"workload": f"{describe(w, info)}; projection at hidden {hid}, "
                                  f"{w.hq}/{w.hkv} heads of {w.d}", "rows": N + NB, "hidden": hid,
                      "out_features": nout, "flop_per_step": flop},
           "pct_of_peak": 100.0 * flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "roofline": {"kernel": "qkv_project", "bound": "mfma",
                        "achieved": flop / (kms * 1e-3) / 1e12 if kms else None,
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": flop / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if kms else None,
                        "traffic": None, "algorithmic_bytes": byt},
           "cpu_baseline": None, "kernels": {"qkv_project": {"launches_per_step": n / args.steps,
                                                             "ms_per_step": kms}}}
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="long256k", choices=workloads.ALL)
    ap.add_argument("--tokens", type=int, default=0,
                    help="with the long256k workload: another sequence length (same CP degree, "
                         "TTT depth and heads), for length sweeps")
    ap.add_argument("--cpu-anchors", type=int, default=10,
                    help="anchors in the CPU-oracle sample (0 skips the CPU baseline)")
    ap.add_argument("--no-profile", action="store_true", help="skip per-kernel event timing")
    ap.add_argument("--mfma-probe-iters", type=int, default=200000,
                    help="iterations of the matrix-core rate probe run after the timed steps "
                         "(0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--stage", default="attention", choices=["attention", "proj"],
                    help="proj: time the draft-layer projection (ba_qkv_project) of the "
                         "workload's main and branch rows instead, at --hidden")
    ap.add_argument("--hidden", type=int, default=4096,
                    help="model width of the projection stage (Qwen3-8B: 4096)")
    ap.add_argument("--walk", default="auto", choices=["auto", "segments", "runs"],
                    help="key walk of the forward and dQ kernels (auto: chosen by chunk size)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp8"],
                    help="fp8: Q/K/Qb/Kb as fp8 E4M3, V bf16; a step is the forward unless "
                         "--fp8-step fwd+bwd (the metric and peak change accordingly)")
    ap.add_argument("--fp8-step", default="fwd", choices=["fwd", "fwd+bwd"],
                    help="what one fp8 step runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the "
              "library computes one context-parallel rank's share on one GPU, with the other "
              "ranks' K/V shards resident in its memory.", file=sys.stderr)
        sys.exit(2)

    import torch
    import branch_attention_speculative_amd as ba
    if not os.path.exists(ba.LIB_PATH):
        from branch_attention_speculative_amd import build as _b
        _b.build()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    w = workloads.make(args.workload)
    if args.tokens:
        if args.workload != "long256k":
            print("--tokens applies to the long256k workload only", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, name=f"ttt{args.tokens}", seqlens=[args.tokens])
    fp8 = args.dtype == "fp8"
    # a step is fwd+bwd for bf16 (every workload); for fp8 it is the forward,
    # or fwd+bwd with --fp8-step fwd+bwd
    if fp8:
        w = dataclasses.replace(w, dtype="fp8", bwd=args.fp8_step == "fwd+bwd")
    else:
        w = dataclasses.replace(w, bwd=True)
    plan = ba.Plan(w.seqlens, w.C, w.r, w.kind, w.depth_or_block, w.anchors, w.branch_lens,
                   w.hq, w.hkv, w.d, w.dtype).upload()
    plan.set_walk(args.walk)
    info = plan.info
    N, NB = info["n_local_rows"], info["n_branch_rows"]
    print(f"[bench] {describe(w, info)}", file=sys.stderr, flush=True)
    if args.stage == "proj":
        return bench_proj(args, ba, torch, w, plan)
    raw = workloads.draw(w, N, NB, names=workloads.TENSOR_ORDER if w.bwd else
                         ["q", "k", "v", "qb", "kb", "vb"])

    def dev(a):
        if a.dtype == np.uint8:  # fp8 E4M3 codes
            return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
        if a.dtype == np.uint16:  # bf16 bits
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    T = {k: dev(v) for k, v in raw.items()}
    ws_f = torch.empty(max(info["ws_fwd_bytes"], 1), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(info["ws_bwd_bytes"], 1), dtype=torch.uint8, device="cuda")
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    def step():
        o, lse, ob, lseb = ba.fwd(plan, T["q"], T["k"], T["v"], T["qb"], T["kb"], T["vb"],
                                  workspace=ws_f)
        if not w.bwd:
            return o, lse, ob, lseb
        return ba.bwd(plan, T["q"], T["k"], T["v"], T["qb"], T["kb"], T["vb"], o, lse, ob, lseb,
                      T["do"], T["dob"], workspace=ws_b)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    if not args.no_profile:
        ba.profile_enable(True, max_launches=16 * args.steps + 16)
        ba.profile_read()  # reset
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    kern = ba.profile_read() if not args.no_profile else {}
    if not args.no_profile:
        ba.profile_enable(False)
    print(f"[bench] timed {args.steps} steps: {ms:.2f} ms/step (wall {wall:.2f} s)", file=sys.stderr,
          flush=True)

    pairs = info["pairs_total"]
    pairs_main_keys = info["pairs_main"] + info["pairs_prefix"]
    flop_step = pairs * w.hq * w.d * (4 + (10 if w.bwd else 0))
    tflops = flop_step / (ms * 1e-3) / 1e12
    if fp8:
        peak = PEAK_FP8_STEP_TFLOPS if w.bwd else PEAK_FP8_QK_BF16_PV_TFLOPS
    else:
        peak = PEAK_BF16_TFLOPS
    kernels = {}
    for name, (n, tot) in kern.items():
        avg = tot / max(n, 1)
        entry = {"launches_per_step": n / args.steps, "avg_ms": avg, "share": tot / (ms * args.steps)}
        if name in KERNEL_FLOP_PER_PAIR_D:
            f = KERNEL_FLOP_PER_PAIR_D[name] * w.d * pairs_main_keys * w.hq
            entry["algorithmic_tflop_per_launch"] = f / 1e12
            entry["achieved_tflops"] = f / (avg * 1e-3) / 1e12
        kernels[name] = entry
    roof = None
    if kernels:
        dom = max((k for k in kernels if k in KERNEL_FLOP_PER_PAIR_D),
                  key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches_per_step"])
        ach = kernels[dom]["achieved_tflops"]
        # each kernel against the peak of its own products: only the forward
        # mixes fp8 and bf16 products in an fp8 plan
        kpeak = PEAK_FP8_QK_BF16_PV_TFLOPS if fp8 and dom == "fwd_ring" else PEAK_BF16_TFLOPS
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": kpeak,
                "unit": "TFLOP/s", "frac": ach / kpeak,
                "traffic": None if fp8 else read_traffic(dom, w.name)}
    probe = None
    if args.mfma_probe_iters > 0:
        # what the matrix cores sustain on register operands on this part, zero
        # and random data (the part is power-limited), after the timed region
        probe = {"zero_operands_tflops": ba.probe_mfma(False, args.mfma_probe_iters),
                 "random_operands_tflops": ba.probe_mfma(True, args.mfma_probe_iters),
                 "iters": args.mfma_probe_iters}
        if roof is not None:
            probe["dominant_kernel_frac_of_random"] = roof["achieved"] / probe["random_operands_tflops"]
    cpu = None
    if args.cpu_anchors > 0:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, info, raw, args.cpu_anchors)
    out = {
        "metric": (METRIC_FP8_STEP if w.bwd else METRIC_FP8) if fp8 else METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": describe(w, info), "tokens": int(sum(w.seqlens)),
                   "cp_degree": w.C, "cp_rank": w.r, "local_rows": N, "branch_rows": NB,
                   "pairs_per_head": pairs, "flop_per_step": flop_step,
                   "key_walk": "run list" if info["run_walk"] else "segments"},
        "pct_of_peak": 100.0 * tflops / peak,
        "roofline": roof,
        "cpu_baseline": cpu,
        "mfma_probe": probe,
        "kernels": kernels,
        "wall_s": wall,
    }
    if kernels:
        # forward and backward separately, from the per-kernel event times
        fwd_ms = sum(k["avg_ms"] * k["launches_per_step"] for n, k in kernels.items()
                     if n.startswith("fwd"))
        bwd_ms = sum(k["avg_ms"] * k["launches_per_step"] for n, k in kernels.items()
                     if n.startswith("bwd"))
        f_fwd, f_bwd = pairs * w.hq * w.d * 4, pairs * w.hq * w.d * 10
        out["split"] = {"fwd_ms": fwd_ms, "bwd_ms": bwd_ms if w.bwd else None,
                        "fwd_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12 if fwd_ms else None,
                        "bwd_tflops": f_bwd / (bwd_ms * 1e-3) / 1e12 if (bwd_ms and w.bwd) else None}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
