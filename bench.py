"""Benchmark: chunked gated linear attention forward + backward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]
python bench.py --workload conv   (the short depthwise causal convolution)
python bench.py --workload norm_gate   (the output per-head RMSNorm x swish gate)
python bench.py --workload delta   (the gated delta rule, chunked WY/UT form)
python bench.py --workload c3 --fused   (q, k, v read in place from one projection
                                          tensor, one fused gradient written)

A step is one gla_fwd followed by one gla_bwd (the whole hot path) over one
batch of seeded synthetic inputs already resident in device memory.  The
default workload is the Mamba-2/SSD shape: scalar decay, fp32, B=4, T=8192,
8 heads in 2 q/k groups, d_k = d_v = 128, chunk 64.  Prints one JSON line.

The roofline object is for gla_bwd, the dominant call of the step: its
algorithmic work divided by its mean duration, timed with HIP events on the
stream the library launches on, against the roofline that binds the path (HBM,
or the matrix cores the products run on: bf16 for bf16 inputs, three bf16
products per fp32 product on the split-bf16 fp32 path).  A default run also
times c3, c4, c5a and c5b in the same process ("also").  The cpu_baseline
object times the fp64 CPU oracle on a bounded sample of the same workload (one
batch row, repeated for about 10 s on all host threads; and one thread on 1024
tokens of that row).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILE = {w: "%s_kernels.md" % w for w in ("c2", "c3", "c4", "c5a", "c5b", "c3f", "conv", "norm_gate", "delta")}


def source_hash():
    """sha256 (first 16 hex) of the HIP sources, as recorded in profile summaries."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "ssm_recurrence_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, key="traffic_bytes_per_gla_bwd"):
    """HBM bytes per backward call (gla_bwd, or gla_conv_bwd: `key`) from the
    committed rocprofv3 counter summary, or None when there is none or the
    kernels changed since it was taken."""
    name = PROFILE.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in (key, "source_hash"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    if vals.get("source_hash") != source_hash() or key not in vals:
        return None
    return float(vals[key])


PEAK = {"hbm": 8000.0,            # GB/s
        "mfma_f32": 157.3,        # TFLOP/s, dense fp32 matrix cores
        "mfma_bf16": 2500.0,      # TFLOP/s, dense bf16 matrix cores
        "valu_f32": 157.3}        # TFLOP/s, fp32 vector ALUs


def algorithmic(case):
    """Algorithmic work of one fwd and one bwd (bytes the method must move,
    FLOPs with the causal half of the chunk products), per the counting used
    for the rooflines: inputs and outputs at their storage dtype, fp32 states."""
    B, T, H, Hqk, dk, dv, Cc = case.B, case.T, case.H, case.H_qk, case.d_k, case.d_v, case.chunk
    es = 2 if case.dtype.__repr__().endswith("bfloat16") else 4
    gw = dk if case.gate == "vector" else 1
    qk = B * T * Hqk * dk * es
    vv = B * T * H * dv * es
    gg = B * T * H * gw * es
    st = B * H * dk * dv * 4
    seg = B * T * 4 if case.segment_ids is not None else 0
    h0 = st if case.h0 is not None else 0
    dhT = st if case.dhT is not None else 0
    fwd_bytes = 2 * qk + vv + gg + h0 + seg + vv + st          # read q k v g (h0, seg); write o, hT
    bwd_bytes = (2 * qk + vv + gg + vv + h0 + dhT + seg         # read q k v g dO (h0 dhT seg)
                 + 2 * qk + vv + gg + (st if case.h0 is not None else 0))  # write dq dk dv dg (dh0)
    th = B * T * H
    fwd_flops = th * (2 * Cc * dk + 2 * dk * dv + 2 * dk * dv)   # intra (causal half) + readout + update
    bwd_flops = th * (4 * Cc * dk + 8 * dk * dv)
    return dict(fwd_bytes=fwd_bytes, bwd_bytes=bwd_bytes, fwd_flops=fwd_flops, bwd_flops=bwd_flops)


def split_bf16_path(case):
    """fp32 inputs whose products run as three bf16 products of split operands on
    the bf16 matrix cores (scalar gate, d_k = d_v = 128)."""
    import torch
    return (case.dtype == torch.float32 and case.gate == "scalar" and case.d_k == 128
            and case.d_v == 128)


def bound_time(case, nbytes, flops):
    """(kind, seconds) of the roofline that binds this work on this path: HBM at
    8 TB/s against the matrix cores the products actually run on (bf16 inputs:
    bf16 cores; split-bf16 fp32: three bf16 products per fp32 product; other
    fp32: the fp32 cores)."""
    import torch
    t_hbm = nbytes / (PEAK["hbm"] * 1e9)
    if case.dtype == torch.bfloat16:
        t_mma = flops / (PEAK["mfma_bf16"] * 1e12)
    elif split_bf16_path(case):
        t_mma = 3 * flops / (PEAK["mfma_bf16"] * 1e12)
    else:
        t_mma = flops / (PEAK["mfma_f32"] * 1e12)
    return ("hbm", t_hbm) if t_hbm >= t_mma else ("mfma", t_mma)


def copy_bandwidth(dev, mib=1024, reps=5):
    """Device-to-device copy rate (GB/s, bytes read + written) of a torch copy."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        b.copy_(a)
    ev[1].record()
    torch.cuda.synchronize()
    sec = ev[0].elapsed_time(ev[1]) / 1000.0 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n * 4 / sec / 1e9


def time_gla(name, steps, warmup, cold=0, fused=False, split=0, saved=True):
    """One gla_fwd + one gla_bwd per step on workload `name`, inputs resident in
    device memory: event-timed fwd and bwd (mean and median), wall time per
    step, and (cold > 0) the median of `cold` steps after a 512 MB cache flush."""
    import torch
    from ssm_recurrence_amd import binding as gb
    from ssm_recurrence_amd.inputs import workload

    dev = torch.device("cuda:0")
    case_cpu = workload(name)
    case = case_cpu.to(dev)
    prob = gb.problem_of(case.q, case.v, case.g, case.gate, case.chunk, split)
    B, T, H, dk, dv = case.B, case.T, case.H, case.d_k, case.d_v
    o = torch.empty((B, T, H, dv), dtype=case.dtype, device=dev)
    hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    dq, dk_, dv_, dg = (torch.empty_like(case.q), torch.empty_like(case.k),
                        torch.empty_like(case.v), torch.empty_like(case.g))
    W = None
    if fused:
        # the projection output X = q | k | v and one gradient buffer of its shape
        W = 2 * case.H_qk * dk + H * dv
        X = torch.empty((B, T, W), dtype=case.dtype, device=dev)
        dX = torch.empty_like(X)
        views = gb.fused_views(X, case.H_qk, dk, H, dv)
        for view, src in zip(views, (case.q, case.k, case.v)):
            view.copy_(src)
        packed = dict(q=case.q, k=case.k, v=case.v, dq=dq, dk=dk_, dv=dv_)
        case.q, case.k, case.v = views
        dq, dk_, dv_ = gb.fused_views(dX, case.H_qk, dk, H, dv)
        prob.ld_qk = prob.ld_v = prob.ld_dqk = prob.ld_dv = W
    dh0 = torch.empty_like(case.h0) if case.h0 is not None else None
    if saved:
        # the forward stores the per-chunk states for the backward in one shared
        # workspace (GLA_SAVE_STATES); the inputs never change, so one generation
        prob.flags, prob.generation = gb.GLA_SAVE_STATES, 1
        nf = nb = gb.workspace_size(prob, True)
        wsf = wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    else:
        nf, nb = gb.workspace_size(prob, False), gb.workspace_size(prob, True)
        wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device=dev)
        wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = gb.ctypes.c_void_p(stream.cuda_stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        gb.fwd_into(prob, case.q, case.k, case.v, case.g, case.h0, case.segment_ids, o, hT, wsf,
                    nf, sp)
        if ev is not None:
            ev[1].record(stream)
        gb.bwd_into(prob, case.q, case.k, case.v, case.g, case.h0, case.segment_ids, case.dO,
                    case.dhT, dq, dk_, dv_, dg, dh0, wsb, nb, sp)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    med = lambda xs: 1000.0 * sorted(xs)[len(xs) // 2]
    r = dict(case=case_cpu, ms_per_step=(t1 - t0) * 1000.0 / steps,
             fwd_us=1000.0 * sum(fwd_ms) / len(fwd_ms), bwd_us=1000.0 * sum(bwd_ms) / len(bwd_ms),
             fwd_med=med(fwd_ms), bwd_med=med(bwd_ms), cold_f=[], cold_b=[], W=W, copies_us=None)

    # cold caches: 512 MB written between steps evicts L2 and the MALL (untimed)
    if cold > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for i in range(cold):
            flush.fill_(i & 0xFF)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            step(ev)
            torch.cuda.synchronize()
            r["cold_f"].append(ev[0].elapsed_time(ev[1]))
            r["cold_b"].append(ev[1].elapsed_time(ev[2]))
        del flush

    # what the packed layout would add around each step: q, k, v split out of the
    # projection, and dq | dk | dv concatenated into its gradient (timed apart)
    if fused:
        def copies():
            packed["q"].copy_(case.q)
            packed["k"].copy_(case.k)
            packed["v"].copy_(case.v)
            torch.cat([packed[n].flatten(2) for n in ("dq", "dk", "dv")], dim=2, out=dX)
        copies()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            copies()
        ev[1].record(stream)
        torch.cuda.synchronize()
        r["copies_us"] = 1000.0 * ev[0].elapsed_time(ev[1]) / steps
    del case, o, hT, dq, dk_, dv_, dg, dh0, wsf, wsb
    torch.cuda.empty_cache()
    return r


def states_note(case, saved):
    """What the backward does for the per-chunk states (GLA_SAVE_STATES stores them
    only for the scalar gate at 128 x 128; other problems recompute them)."""
    if not saved:
        return "recomputed by the backward (separate workspaces)"
    if case.gate == "scalar" and case.d_k == 128 and case.d_v == 128:
        return "stored by the forward for the backward (GLA_SAVE_STATES, one workspace)"
    return "recomputed by the backward (one workspace; GLA_SAVE_STATES stores none for this problem)"


def gla_roofline(case, fwd_us, bwd_us, copy_gbs=None):
    """Roofline of gla_bwd (the dominant call) and of the whole step, against the
    bound that binds the path (bound_time); fp32 paths also report the fraction
    of the fp32 matrix-core peak their FLOPs would reach."""
    import torch
    alg = algorithmic(case)
    kind, tb = bound_time(case, alg["bwd_bytes"], alg["bwd_flops"])
    _, ts = bound_time(case, alg["fwd_bytes"] + alg["bwd_bytes"], alg["fwd_flops"] + alg["bwd_flops"])
    sec = bwd_us * 1e-6
    if kind == "hbm":
        roof = {"bound": "hbm", "achieved": round(alg["bwd_bytes"] / sec / 1e9, 3),
                "peak": PEAK["hbm"], "unit": "GB/s"}
    else:
        mult = 3 if split_bf16_path(case) else 1
        peak = PEAK["mfma_f32"] if (case.dtype == torch.float32 and mult == 1) else PEAK["mfma_bf16"]
        roof = {"bound": "mfma", "achieved": round(mult * alg["bwd_flops"] / sec / 1e12, 3),
                "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = round(tb / sec, 4)
    roof["step_frac"] = round(ts / ((fwd_us + bwd_us) * 1e-6), 4)
    roof["algorithmic_bytes"] = round(alg["bwd_bytes"] / 1e6, 1)
    roof["algorithmic_gflop"] = round(alg["bwd_flops"] / 1e9, 2)
    if copy_gbs:
        roof["copy_gbs"] = round(copy_gbs, 1)
        roof["copy_frac"] = round(alg["bwd_bytes"] / sec / 1e9 / copy_gbs, 4)
    if case.dtype == torch.float32:
        # the fp32 FLOPs against the fp32 matrix cores (the split-bf16 path does not use them)
        roof["fp32_mfma_frac"] = round(alg["bwd_flops"] / sec / 1e12 / PEAK["mfma_f32"], 4)
        roof["step_fp32_mfma_frac"] = round((alg["fwd_flops"] + alg["bwd_flops"])
                                            / ((fwd_us + bwd_us) * 1e-6) / 1e12 / PEAK["mfma_f32"], 4)
    if split_bf16_path(case):
        roof["products"] = "fp32 as three bf16 products of split operands (bf16 matrix cores)"
    return roof


def cpu_baseline(case, single_seconds=5.0):
    """The fp64 oracle on the host cores over a bounded sample: batch row 0, every
    head, the whole sequence, fwd + bwd repeated for about 10 s on all threads in
    the affinity mask; plus one thread on the first 1024 tokens of that row."""
    import oracle
    threads = oracle.default_threads()
    s = case
    T, H = s.T, s.H

    def run(sl, tsl, nthreads, budget):
        cut = lambda x: None if x is None else x[sl][:, tsl].contiguous()
        st = lambda x: None if x is None else x[sl].contiguous()
        args = (cut(s.q), cut(s.k), cut(s.v), cut(s.g))
        seg = None if s.segment_ids is None else s.segment_ids[sl][:, tsl].contiguous()
        c0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - c0 < budget:
            oracle.fwd(*args, st(s.h0), seg, gate=s.gate, threads=nthreads)
            oracle.bwd(*args, cut(s.dO), st(s.h0), seg, st(s.dhT), gate=s.gate, threads=nthreads)
            reps += 1
        return reps, time.perf_counter() - c0

    reps, sec = run(slice(0, 1), slice(0, T), threads, 10.0)
    n1 = min(T, 1024)
    reps1, sec1 = run(slice(0, 1), slice(0, n1), 1, single_seconds)
    return {"value": round(reps * T / sec, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "batch row 0 of the workload (%d tokens x %d heads), fwd+bwd, %d times in %.1f s"
                      % (T, H, reps, sec),
            "single_thread": {"value": round(reps1 * n1 / sec1, 1), "unit": "tokens/s", "cores": 1,
                              "sample": "tokens 0..%d of batch row 0, every head, fwd+bwd, %d times "
                                        "in %.1f s" % (n1 - 1, reps1, sec1)}}


# workloads timed beside the headline one in a default run (no CPU leg)
ALSO = ["c3", "c4", "c5a", "c5b"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=3,
                    help="extra untimed-region steps after a 512 MB cache flush (median reported)")
    ap.add_argument("--fused", action="store_true",
                    help="q, k, v as views of one [B, T, 2*H_qk*d_k + H*d_v] projection tensor, "
                         "dq, dk, dv written into one fused gradient of that shape")
    ap.add_argument("--split", type=int, default=0,
                    help="sequence pieces per (b, h); 0 = the library's own choice")
    ap.add_argument("--states", choices=("saved", "recompute"), default="saved",
                    help="saved: the forward stores the per-chunk states for the backward "
                         "(GLA_SAVE_STATES, one shared workspace); recompute: the backward "
                         "recomputes them")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads timed beside the main one (default: %s for "
                         "the default workload, none otherwise; 'none' for none)" % ",".join(ALSO))
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from ssm_recurrence_amd import binding as gb  # noqa: F401  (fails loudly without the library)
    from ssm_recurrence_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "conv":
        conv_main(args)
        return
    if args.workload == "norm_gate":
        norm_gate_main(args)
        return
    if args.workload == "delta":
        delta_main(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_gbs = copy_bandwidth(dev)
    saved = args.states == "saved"
    r = time_gla(args.workload, args.steps, args.warmup, args.cold, args.fused, args.split, saved)
    case = r["case"]
    B, T, H, dk, dv = case.B, case.T, case.H, case.d_k, case.d_v
    fwd_us, bwd_us = r["fwd_us"], r["bwd_us"]
    value = B * T / (r["ms_per_step"] / 1000.0)
    roof = gla_roofline(case, fwd_us, bwd_us, copy_gbs)
    traffic = measured_traffic(args.workload + ("f" if args.fused else ""))
    roof["traffic"] = None if traffic is None else round(traffic / 1e6, 1)
    roof["traffic_unit"] = "MB per gla_bwd call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["kernel"] = "gla_bwd (all its kernels, one call)"
    cpu = None if args.no_cpu_baseline else cpu_baseline(case)
    bf16 = case.dtype == torch.bfloat16
    med = lambda xs: 1000.0 * sorted(xs)[len(xs) // 2]

    out = {
        "metric": "fwd+bwd µs and tokens/s for chunked GLA/SSD at d=128, % of MFMA/HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
        "us_fwd": round(fwd_us, 1), "us_bwd": round(bwd_us, 1),
        "us_fwd_bwd": round(fwd_us + bwd_us, 1),
        "us_fwd_median": round(r["fwd_med"], 1), "us_bwd_median": round(r["bwd_med"], 1),
        "us_fwd_cold": round(med(r["cold_f"]), 1) if r["cold_f"] else None,
        "us_bwd_cold": round(med(r["cold_b"]), 1) if r["cold_b"] else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic (seeded)",
        "config": {"workload": "%s: %s" % (args.workload, WORKLOADS[args.workload]),
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv,
                   "chunk": case.chunk, "split": args.split, "parallelism": "single GPU",
                   "states": states_note(case, saved),
                   "layout": ("q, k, v read from one [B, T, %d] projection tensor; one fused "
                              "gradient" % r["W"]) if args.fused else "packed q, k, v"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.fused:
        out["us_layout_copies_avoided"] = round(r["copies_us"], 1)

    also = args.also
    if also is None:
        also = ",".join(ALSO) if (args.workload == "c2" and not args.fused and args.split == 0) else "none"
    others = {}
    for name in [x for x in also.split(",") if x and x != "none"]:
        o = time_gla(name, args.steps, args.warmup, saved=saved)
        c = o["case"]
        rf = gla_roofline(c, o["fwd_us"], o["bwd_us"], copy_gbs)
        others[name] = {"workload": WORKLOADS[name],
                        "us_fwd": round(o["fwd_us"], 1), "us_bwd": round(o["bwd_us"], 1),
                        "us_fwd_bwd": round(o["fwd_us"] + o["bwd_us"], 1),
                        "tokens_per_s": round(c.B * c.T / (o["ms_per_step"] / 1000.0), 1),
                        "bound": rf["bound"], "bwd_frac": rf["frac"], "step_frac": rf["step_frac"],
                        "copy_frac": rf.get("copy_frac")}
    if others:
        out["also"] = others
    print(json.dumps(out))


def conv_main(args):
    """The short depthwise causal convolution (K = 4, bias, SiLU) at the page's
    benchmark shape: one gla_conv_fwd and one gla_conv_bwd per step."""
    import torch
    from ssm_recurrence_amd import binding as gb
    from ssm_recurrence_amd.inputs import conv_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case_cpu = conv_workload()
    c = case_cpu.to(dev)
    B, T, C = c.x.shape
    K = c.w.shape[0]
    prob = gb.conv_problem(c.x, K)
    y, dx = torch.empty_like(c.x), torch.empty_like(c.x)
    dw, db = torch.empty_like(c.w), torch.empty(C, dtype=torch.float32, device=dev)
    n = gb.conv_workspace_size(prob)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = gb.ctypes.c_void_p(stream.cuda_stream)
    lib = gb.load()
    P = gb.ctypes.byref(prob)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = lib.gla_conv_fwd(P, gb._p(c.x), gb._p(c.w), gb._p(c.bias), gb._p(y), sp)
        if ev is not None:
            ev[1].record(stream)
        rc |= lib.gla_conv_bwd(P, gb._p(c.x), gb._p(c.w), gb._p(c.bias), gb._p(c.dy), gb._p(dx),
                               gb._p(dw), gb._p(db), gb._p(ws), ws.numel(), sp)
        if ev is not None:
            ev[2].record(stream)
        if rc:
            raise RuntimeError("gla_conv_* failed: %d" % rc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    fwd_us = 1000.0 * sum(fwd_ms) / len(fwd_ms)
    bwd_us = 1000.0 * sum(bwd_ms) / len(bwd_ms)
    # algorithmic bytes: forward reads x, writes y; backward reads x, dy, writes dx
    # (taps, bias and their gradients are C * (2K + 2) * 4 bytes, included)
    es = c.x.element_size()
    par = C * (2 * K + 2) * 4
    fwd_bytes = 2 * B * T * C * es + par
    bwd_bytes = 3 * B * T * C * es + par
    achieved = bwd_bytes / (bwd_us * 1e-6) / 1e9
    traffic = measured_traffic("conv", "traffic_bytes_per_gla_conv_bwd")
    roof = {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK["hbm"], "unit": "GB/s",
            "frac": round(achieved / PEAK["hbm"], 4),
            "traffic": None if traffic is None else round(traffic / 1e6, 1),
            "traffic_unit": "MB per gla_conv_bwd call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": round(bwd_bytes / 1e6, 1),
            "kernel": "gla_conv_bwd (its two kernels, one call)",
            "step_frac": round((fwd_bytes + bwd_bytes) / ((fwd_us + bwd_us) * 1e-6) / 1e9 / PEAK["hbm"], 4)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.conv as oc
        s = case_cpu
        c0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - c0 < 10.0:
            oc.conv_fwd(s.x, s.w, s.bias)
            oc.conv_bwd(s.x, s.w, s.bias, s.dy)
            reps += 1
        c1 = time.perf_counter()
        cpu = {"value": round(reps * B * T / (c1 - c0), 1), "unit": "tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": "the whole workload (%d rows x %d steps x %d channels), fwd+bwd in numpy "
                         "fp64 on one thread, %d times in %.1f s" % (B, T, C, reps, c1 - c0)}
    out = {
        "metric": "fwd+bwd µs and tokens/s for the short depthwise causal convolution (K=4, bias, SiLU), % of HBM roofline",
        "value": round(B * T / (ms_per_step / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "us_fwd": round(fwd_us, 1), "us_bwd": round(bwd_us, 1), "us_fwd_bwd": round(fwd_us + bwd_us, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": "conv: depthwise causal conv K=4 + bias + SiLU, bf16, B=8 T=4096 C=2048",
                   "global_batch": B, "seq_len": T, "channels": C, "taps": K,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))



def norm_gate_main(args):
    """The output norm and gate (per-head RMSNorm x swish gate) at the layer shape
    of the page's benchmarks: one gla_norm_gate_fwd and one gla_norm_gate_bwd per step."""
    import torch
    from ssm_recurrence_amd import binding as gb
    from ssm_recurrence_amd.inputs import norm_gate_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case_cpu = norm_gate_workload()
    c = case_cpu.to(dev)
    B, T, H, d = c.o.shape
    prob = gb.norm_gate_problem(c.o, c.eps)
    y, d_o, dz = torch.empty_like(c.o), torch.empty_like(c.o), torch.empty_like(c.o)
    dgamma = torch.empty_like(c.gamma)
    n = gb.norm_gate_workspace_size(prob)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = gb.ctypes.c_void_p(stream.cuda_stream)
    lib = gb.load()
    P = gb.ctypes.byref(prob)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = lib.gla_norm_gate_fwd(P, gb._p(c.o), gb._p(c.z), gb._p(c.gamma), gb._p(y), sp)
        if ev is not None:
            ev[1].record(stream)
        rc |= lib.gla_norm_gate_bwd(P, gb._p(c.o), gb._p(c.z), gb._p(c.gamma), gb._p(c.dy), gb._p(d_o),
                                    gb._p(dz), gb._p(dgamma), gb._p(ws), ws.numel(), sp)
        if ev is not None:
            ev[2].record(stream)
        if rc:
            raise RuntimeError("gla_norm_gate_* failed: %d" % rc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    fwd_us = 1000.0 * sum(fwd_ms) / len(fwd_ms)
    bwd_us = 1000.0 * sum(bwd_ms) / len(bwd_ms)
    # algorithmic bytes: forward reads o, z and writes y; backward reads o, z, dy
    # and writes do, dz (gamma and dgamma, d * 4 bytes each, included)
    es = c.o.element_size()
    elems = B * T * H * d
    fwd_bytes = 3 * elems * es + d * 4
    bwd_bytes = 5 * elems * es + 2 * d * 4
    achieved = bwd_bytes / (bwd_us * 1e-6) / 1e9
    traffic = measured_traffic("norm_gate", "traffic_bytes_per_gla_norm_gate_bwd")
    roof = {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK["hbm"], "unit": "GB/s",
            "frac": round(achieved / PEAK["hbm"], 4),
            "traffic": None if traffic is None else round(traffic / 1e6, 1),
            "traffic_unit": "MB per gla_norm_gate_bwd call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": round(bwd_bytes / 1e6, 1),
            "kernel": "gla_norm_gate_bwd (its two kernels, one call)",
            "step_frac": round((fwd_bytes + bwd_bytes) / ((fwd_us + bwd_us) * 1e-6) / 1e9 / PEAK["hbm"], 4)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.norm_gate as on
        s = case_cpu
        o0, z0, dy0 = s.o[0], s.z[0], s.dy[0]  # batch row 0: T tokens, every head
        c0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - c0 < 10.0:
            on.norm_gate_fwd(o0, z0, s.gamma, s.eps)
            on.norm_gate_bwd(o0, z0, s.gamma, dy0, s.eps)
            reps += 1
        c1 = time.perf_counter()
        cpu = {"value": round(reps * T / (c1 - c0), 1), "unit": "tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": "batch row 0 (%d steps x %d heads x %d channels), fwd+bwd in numpy fp64 on "
                         "one thread, %d times in %.1f s" % (T, H, d, reps, c1 - c0)}
    out = {
        "metric": "fwd+bwd µs and tokens/s for the output per-head RMSNorm x swish gate, % of HBM roofline",
        "value": round(B * T / (ms_per_step / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "us_fwd": round(fwd_us, 1), "us_bwd": round(bwd_us, 1), "us_fwd_bwd": round(fwd_us + bwd_us, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": "norm_gate: per-head RMSNorm x swish gate, bf16, B=8 T=4096 H=16 d=128, "
                               "eps=%g" % c.eps,
                   "global_batch": B, "seq_len": T, "heads": H, "d": d, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def delta_flops(T, C, dk, dv):
    """FLOPs of the chunked WY/UT gated delta rule per (b, h): dense products of
    each chunk as the method forms them.  The backward reuses the forward's
    per-chunk factors (the workspace it is handed) and recomputes the states
    entering the chunks, as a backward that keeps only chunk-boundary states must."""
    nc = (T + C - 1) // C
    c2k, c2v, cdd, c3 = 2 * C * C * dk, 2 * C * C * dv, 2 * C * dk * dv, 2 * C ** 3
    prep = 2 * c2k + c2v + c2k + c3 / 3           # K K^T, U, W, Q K^T, the inverse
    state = 3 * cdd + c2v                          # W S0, (gamma Q) S0, Kt^T Wv; P Wv
    fwd = prep + state
    dstate = c2v + 3 * cdd                         # P^T dO; Kt dS1, (gamma Q)^T dO, W^T dWv
    grad = (c2k + 3 * cdd                          # K K^T; dO S0^T, Wv dS1^T, dWv S0^T
            + c2v + 2 * c2k                        # dO Wv^T; (dP M) K, (dP M)^T Q
            + c2v + c2k + c2v + c2k                # dT (two), T^T dWv, T^T dW
            + 2 * c3 + 2 * c2k)                    # dA = -T^T dT T^T; (dG + dG^T) K
    bwd = cdd + dstate + grad                      # (the state pass without readout: W S0)
    return nc * fwd, nc * bwd


def delta_main(args):
    """The gated delta rule at the pages' Gated DeltaNet benchmark layout (bf16,
    batch 4, 8 heads, chunk 64, d = 128) at T = 4096: one gla_delta_fwd and one
    gla_delta_bwd per step, the backward handed the forward's workspace
    (GLA_DELTA_WS_FROM_FWD), as the autograd wrapper does."""
    import torch
    from ssm_recurrence_amd import binding as gb
    from ssm_recurrence_amd.inputs import delta_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case_cpu = delta_workload()
    c = case_cpu.to(dev)
    B, T, H, dk = c.q.shape
    dv = c.v.shape[3]
    # the backward may reuse what the forward left in ws: its per-chunk factors and
    # states (same inputs, same generation; the flag on both calls)
    prob = gb.delta_problem(c.q, c.v, gb.GLA_DELTA_WS_FROM_FWD, 1)
    prob_b = prob
    o = torch.empty_like(c.v)
    hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    dq, dk_, dv_, dg, db = (torch.empty_like(c.q), torch.empty_like(c.k), torch.empty_like(c.v),
                            torch.empty_like(c.g), torch.empty_like(c.beta))
    dh0 = torch.empty_like(c.h0)
    n = gb.delta_workspace_size(prob)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    n2 = gb.delta_workspace_size(prob, True)
    scratch = torch.empty(max(n2, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = gb.ctypes.c_void_p(stream.cuda_stream)
    lib = gb.load()
    P, PB = gb.ctypes.byref(prob), gb.ctypes.byref(prob_b)
    p = gb._p

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = lib.gla_delta_fwd(P, p(c.q), p(c.k), p(c.v), p(c.g), p(c.beta), p(c.h0), p(c.segment_ids),
                               p(o), p(hT), p(ws), ws.numel(), sp)
        if ev is not None:
            ev[1].record(stream)
        rc |= lib.gla_delta_bwd(PB, p(c.q), p(c.k), p(c.v), p(c.g), p(c.beta), p(c.h0), p(c.segment_ids),
                                p(c.dO), p(c.dhT), p(dq), p(dk_), p(dv_), p(dg), p(db), p(dh0), p(ws),
                                ws.numel(), p(scratch), scratch.numel(), sp)
        if ev is not None:
            ev[2].record(stream)
        if rc:
            raise RuntimeError("gla_delta_* failed: %d" % rc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    fwd_us = 1000.0 * sum(fwd_ms) / len(fwd_ms)
    bwd_us = 1000.0 * sum(bwd_ms) / len(bwd_ms)
    ff, fb = delta_flops(T, 64, dk, dv)
    ff, fb = ff * B * H, fb * B * H
    achieved = fb / (bwd_us * 1e-6) / 1e12
    traffic = measured_traffic("delta", "traffic_bytes_per_gla_delta_bwd")
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK["mfma_f32"], "unit": "TFLOP/s",
            "frac": round(achieved / PEAK["mfma_f32"], 4),
            "traffic": None if traffic is None else round(traffic / 1e6, 1),
            "traffic_unit": "MB per gla_delta_bwd call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flops": round(fb / 1e9, 2),
            "kernel": "gla_delta_bwd (its three kernels, one call): fp32 products, mostly on the matrix cores",
            "step_frac": round((ff + fb) / ((fwd_us + bwd_us) * 1e-6) / 1e12 / PEAK["mfma_f32"], 4)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.delta as od
        s = case_cpu
        sl = lambda x: None if x is None else x[0:1, :, 0:1].contiguous()  # (b, h) = (0, 0)
        hs = lambda x: None if x is None else x[0:1, 0:1].contiguous()
        c0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - c0 < 10.0:
            od.delta_fwd(sl(s.q), sl(s.k), sl(s.v), sl(s.g), sl(s.beta), hs(s.h0), None)
            od.delta_bwd(sl(s.q), sl(s.k), sl(s.v), sl(s.g), sl(s.beta), sl(s.dO), hs(s.h0), None, hs(s.dhT))
            reps += 1
        c1 = time.perf_counter()
        cpu = {"value": round(reps * T / H / (c1 - c0), 1), "unit": "tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": "one (batch row, head) of the workload (%d steps), fwd+bwd in numpy fp64 on one "
                         "thread, %d times in %.1f s; tokens/s counts a token as all %d heads" % (T, reps, c1 - c0, H)}
    out = {
        "metric": "fwd+bwd µs and tokens/s for the gated delta rule (chunked WY/UT form), % of fp32 MFMA peak",
        "value": round(B * T / (ms_per_step / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "us_fwd": round(fwd_us, 1), "us_bwd": round(bwd_us, 1), "us_fwd_bwd": round(fwd_us + bwd_us, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": "delta: gated delta rule, bf16, B=4 T=4096 H=8 d_k=d_v=128, chunk 64, h0 and dhT",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv, "chunk": 64,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))

if __name__ == "__main__":
    main()
