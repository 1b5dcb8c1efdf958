"""rocprofv3 summaries of the library's kernels for one bench.py workload.

python3 -m ssm_recurrence_amd.profile --workload c3 [--out gpurun_out/prof_c3] [--md FILE]

Runs bench.py under rocprofv3 as child processes (the profiler wraps python3
itself; this driver never touches the GPU), one pass per counter group:

  trace   --kernel-trace --stats            per-kernel average durations
  fetch   --pmc FETCH_SIZE SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
  write   --pmc WRITE_SIZE
  and the fetch and write passes over the copy-calibration program
  (python3 -m ssm_recurrence_amd.calib), whose byte count is known,

then writes a markdown summary: per kernel the average duration, HBM bytes
read and written per dispatch (counters scaled by the copy's factors), the
achieved HBM rate, and the matrix cores' busy share,
  MFMA busy = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMDs)
(the rocprofiler SDK's MfmaUtil; the per-dispatch GRBM_GUI_ACTIVE of the csv
output is summed over the chip's XCDs, so its maximum is that sum / XCDs).  The summary records the kernel sources'
hash; bench.py reports its traffic figure only while the sources still match.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PASS_TIMEOUT = 240         # seconds per profiler pass

TITLE = {
    "c1": "SSD scalar decay, fp32, B=1 T=256 H=2 d=64, chunk 64",
    "c2": "SSD scalar decay, fp32, B=4 T=8192 H=8 (2 q/k groups) d_k=d_v=128, chunk 64",
    "c3": "GLA vector decay, bf16 inputs / fp32 accumulation, B=4 T=4096 H=16 d_k=d_v=128, chunk 64, h0 and dhT",
    "c4": "SSD scalar decay, bf16, packed documents, B=1 T=65536 H=16 d_k=d_v=128, chunk 64, h0",
    "c5a": "GLA vector decay, bf16, B=1 T=16384 H=16 d_k=d_v=128, chunk 64, h0 and dhT",
    "c5b": "GLA vector decay, bf16, B=8 T=2048 H=16 d_k=d_v=128, chunk 64, h0 and dhT",
    "c3f": "c3 with q, k, v read in place from one [B, T, 3 H d] projection tensor and one fused gradient",
    "conv": "short depthwise causal convolution K=4 + bias + SiLU, bf16, B=8 T=4096 C=2048",
    "norm_gate": "output per-head RMSNorm x swish gate, bf16, B=8 T=4096 H=16 d=128",
    "delta": "gated delta rule (chunked WY/UT), bf16, B=4 T=4096 H=8 d_k=d_v=128, chunk 64",
}
# the library call each kernel belongs to, by workload family
CALLS = {"conv": ("gla_conv_fwd", "gla_conv_bwd"), "norm_gate": ("gla_norm_gate_fwd", "gla_norm_gate_bwd"),
         "delta": ("gla_delta_fwd", "gla_delta_bwd")}


def source_hash():
    """sha256 (first 16 hex) of the HIP sources (the same digest bench.py checks)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def part_of(workload, name):
    """The library calls that launch kernel `name` (empty for torch's own kernels)."""
    if "gla::" not in name and not name.startswith("_ZN3gla"):
        return []
    fwd, bwd = CALLS.get(workload, ("gla_fwd", "gla_bwd"))
    if workload in CALLS:
        # (the delta rule's prepare pass is launched by both calls, the backward's
        # launch exiting when the forward's factors are found: split per dispatch
        # below; its forward state pass is k_delta_state<T, false, D>, "Lb0E" mangled)
        if "fwd" in name or "delta_prep" in name or ("k_delta_state" in name and "Lb0E" in name):
            return [fwd]
        return [bwd]
    if "k_piece_combine" in name:
        return [fwd, bwd]
    if "k_fwd" in name:
        return [fwd]
    if "k_states" in name and "k_states2" not in name:
        # template integers (demangled "..., 128, 1, 128>" or mangled "Li128ELi1ELi128E"):
        # k_states<T, VEC, DK, DV, MODE, NB>, k_states_w<T, DK, DV, MODE>; mode 1 is the
        # forward split's summaries
        ints = re.findall(r"Li(\d+)E", name) if name.startswith("_Z") else \
            re.findall(r"\b(\d+)\b", name[name.find("<"):name.rfind(">") + 1])
        mode = ints[-1] if "k_states_w" in name else ints[-2]
        return [fwd] if mode == "1" else [bwd]
    return [bwd]


def run(cmd, log):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(PASS_TIMEOUT)] + cmd, cwd=ROOT, stdout=f,
                           stderr=subprocess.STDOUT)
    if r.returncode != 0:
        # the profiler may end with a signal after a complete run; its files decide
        print("  (exit status %d; see %s)" % (r.returncode, log), flush=True)
    return r.returncode


def find_csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[0]


def kernel_stats(d):
    """{kernel: (calls, average ns)} from a --stats run."""
    out = {}
    with open(find_csv(d, "kernel_stats.csv")) as f:
        for row in csv.DictReader(f):
            out[row["Name"]] = (int(row["Calls"]), float(row["AverageNs"]))
    return out


def counters(d):
    """{kernel: {counter: [value per dispatch, in dispatch order]}} from a --pmc run."""
    rows = []
    with open(find_csv(d, "counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            rows.append((int(row["Dispatch_Id"]), row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])))
    out = {}
    for _, k, c, v in sorted(rows, key=lambda r: r[0]):
        out.setdefault(k, {}).setdefault(c, []).append(v)
    return out


def dispatch_ns(d):
    """{kernel: [duration in ns per dispatch, in dispatch order]} from a --kernel-trace run."""
    rows = []
    with open(find_csv(d, "kernel_trace.csv")) as f:
        for row in csv.DictReader(f):
            rows.append((int(row["Start_Timestamp"]), row["Kernel_Name"],
                         int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
    out = {}
    for _, k, ns in sorted(rows):
        out.setdefault(k, []).append(ns)
    return out


def gpu_agent(d):
    """(SIMDs, XCDs) of the GPU agent in a run's agent info."""
    with open(find_csv(d, "agent_info.csv")) as f:
        for row in csv.DictReader(f):
            if row.get("Agent_Type") == "GPU":
                return int(row["Simd_Count"]), max(1, int(row["Num_Xcc"]))
    raise ValueError("no GPU agent in " + d)


def mean(xs):
    return sum(xs) / len(xs) if xs else 0.0


def bench_cmd(workload, steps, warmup):
    wl = ["--workload", "c3", "--fused"] if workload == "c3f" else ["--workload", workload]
    return ["python3", "bench.py"] + wl + ["--steps", str(steps), "--warmup", str(warmup), "--cold", "0",
                                           "--no-cpu-baseline", "--also", "none"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", default=None, help="directory for the raw profiler output")
    ap.add_argument("--md", default=None, help="summary file (default profiles/<workload>_kernels.md)")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--summarize-only", action="store_true",
                    help="write the summary from the raw output already in --out (no profiler runs)")
    a = ap.parse_args()
    w = a.workload
    out = a.out or os.path.join(ROOT, "gpurun_out", "prof_" + w)
    md = a.md or os.path.join(ROOT, "profiles", "%s_kernels.md" % w)
    os.makedirs(out, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")
    rp = ["rocprofv3", "--output-format", "csv", "-o", "run", "-d"]
    fetch_ctr = ["FETCH_SIZE", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
    passes = [
        ("trace", rp + [os.path.join(out, "trace"), "--kernel-trace", "--stats", "--"] + bench_cmd(w, a.steps, a.warmup)),
        ("fetch", rp + [os.path.join(out, "fetch"), "--pmc"] + fetch_ctr + ["--"] + bench_cmd(w, 2, 1)),
        ("write", rp + [os.path.join(out, "write"), "--pmc", "WRITE_SIZE", "--"] + bench_cmd(w, 2, 1)),
        ("copy_fetch", rp + [os.path.join(out, "copy_fetch"), "--pmc", "FETCH_SIZE", "--", "python3", "-m",
                             "ssm_recurrence_amd.calib"]),
        ("copy_write", rp + [os.path.join(out, "copy_write"), "--pmc", "WRITE_SIZE", "--", "python3", "-m",
                             "ssm_recurrence_amd.calib"]),
    ]
    if not a.summarize_only:
        for tag, cmd in passes:
            run(cmd, os.path.join(out, tag + ".log"))

    stats = kernel_stats(os.path.join(out, "trace"))
    per_dispatch = dispatch_ns(os.path.join(out, "trace"))
    simds, xcds = gpu_agent(os.path.join(out, "fetch"))
    cf, cw = counters(os.path.join(out, "fetch")), counters(os.path.join(out, "write"))
    # the copy: the largest torch copy dispatch reads and writes the calibration size
    mib = 256
    kib = mib * 1024
    copy_f = max((mean(v["FETCH_SIZE"]) for v in counters(os.path.join(out, "copy_fetch")).values()
                  if "FETCH_SIZE" in v), default=0.0)
    copy_w = max((mean(v["WRITE_SIZE"]) for v in counters(os.path.join(out, "copy_write")).values()
                  if "WRITE_SIZE" in v), default=0.0)
    kf = kib / copy_f if copy_f else float("nan")
    kw = kib / copy_w if copy_w else float("nan")
    launches = a.steps + a.warmup

    rows, per_call = [], {}
    total = sum(ns * n for name, (n, ns) in stats.items() if part_of(w, name))
    fwd_key, bwd_key = CALLS.get(w, ("gla_fwd", "gla_bwd"))
    for name, (calls, ns) in sorted(stats.items(), key=lambda x: -x[1][0] * x[1][1]):
        parts = part_of(w, name)
        if not parts:
            continue
        c1, c2 = cf.get(name, {}), cw.get(name, {})
        rd = mean(c1.get("FETCH_SIZE", [])) * kf * 1024.0       # bytes per dispatch
        wr = mean(c2.get("WRITE_SIZE", [])) * kw * 1024.0
        busy, act = mean(c1.get("SQ_VALU_MFMA_BUSY_CYCLES", [])), mean(c1.get("GRBM_GUI_ACTIVE", []))
        mfma = busy / (act / xcds * simds) if act > 0 else float("nan")
        gbs = (rd + wr) / (ns * 1e-9) / 1e9 if ns > 0 else float("nan")
        # A forward pass launched twice per step: by the forward, and by a backward
        # that finds what the forward stored (that launch exits at once): the
        # forward summaries, the delta rule's prepare pass.  Its dispatches
        # alternate forward, backward in every run.
        both = parts == [fwd_key] and calls == 2 * launches
        rows.append((name, calls, ns / 1000.0, (fwd_key + " + " + bwd_key) if both else " + ".join(parts),
                     rd / 1e6, wr / 1e6, gbs, mfma, ns * calls / total))
        if both:
            dur = per_dispatch.get(name, [])
            for k, key in enumerate((fwd_key, bwd_key)):
                d = per_call.setdefault(key, [0.0, 0.0])
                d[0] += mean(dur[k::2]) / 1000.0
                d[1] += (mean(c1.get("FETCH_SIZE", [])[k::2]) * kf + mean(c2.get("WRITE_SIZE", [])[k::2]) * kw) * 1024.0
            continue
        # per step, each of the calls that launch it gets an equal part of its launches
        per = calls / launches / len(parts)
        for p in parts:
            d = per_call.setdefault(p, [0.0, 0.0])
            d[0] += per * ns / 1000.0
            d[1] += per * (rd + wr)

    lines = []
    lines.append("# %s kernels: %s" % (w, TITLE.get(w, w)))
    lines.append("")
    lines.append("Made by `python3 -m ssm_recurrence_amd.profile --workload %s` (repository root, one MI355X), "
                 "which ran:" % w)
    lines.append("")
    lines.append("```")
    for tag, cmd in passes:
        lines.append("TMPDIR=/tmp " + " ".join(cmd).replace(ROOT + "/", ""))
    lines.append("```")
    lines.append("")
    lines.append("Kernel source hash (sha256 of ssm_recurrence_amd/csrc/*, first 16 hex): `%s`" % source_hash())
    lines.append("")
    lines.append("Copy calibration: torch's copy of %d MiB reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB, "
                 "so bytes = FETCH_SIZE x %.3f KiB and WRITE_SIZE x %.3f KiB." % (mib, copy_f, copy_w, kf, kw))
    lines.append("")
    lines.append("| kernel | calls | avg µs | part of | read MB | written MB | HBM GB/s | MFMA busy | share of time |")
    lines.append("|---|---|---|---|---|---|---|---|---|")
    for name, calls, us, part, rd, wr, gbs, mfma, sh in rows:
        lines.append("| `%s` | %d | %.1f | %s | %.1f | %.1f | %.0f | %.1f %% | %.1f %% |"
                     % (name, calls, us, part, rd, wr, gbs, 100 * mfma, 100 * sh))
    lines.append("")
    lines.append("Per call and step (%d steps profiled; the sum over the kernels a call launches, a kernel "
                 "launched by both calls counted half to each, except a forward pass that the backward "
                 "launches too (exiting at once on what the forward stored), whose dispatches alternate "
                 "between the two calls):" % launches)
    lines.append("")
    for key in sorted(per_call):
        us, nb = per_call[key]
        lines.append("- %s: %.1f µs, %.1f MB of HBM traffic, %.0f GB/s" % (key, us, nb / 1e6, nb / (us * 1e-6) / 1e9))
    lines.append("")
    lines.append("(HBM GB/s: (read + written) / average duration, per kernel.  MFMA busy: the matrix cores' "
                 "busy cycles over the cycles the GPU was active (GRBM_GUI_ACTIVE / %d XCDs) times %d SIMDs.)"
                 % (xcds, simds))
    lines.append("")
    if bwd_key in per_call:
        lines.append("traffic_bytes_per_%s: %.0f" % (bwd_key, per_call[bwd_key][1]))
    lines.append("source_hash: %s" % source_hash())
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", md)


if __name__ == "__main__":
    main()
