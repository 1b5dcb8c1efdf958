"""Copy-kernel calibration for the HBM byte counters.

python -m ssm_recurrence_amd.calib [--mib 256] [--reps 5]

Copies a device buffer of known size with torch's copy kernel; each copy
reads and writes exactly `mib` MiB.  Profiling this command with the
FETCH_SIZE and WRITE_SIZE counters gives the factor between counter readings
and bytes actually moved, which scales the counters of the library's kernels.
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=256)
    ap.add_argument("--reps", type=int, default=5)
    a = ap.parse_args()
    n = a.mib * 1024 * 1024 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copied %d MiB x %d" % (a.mib, a.reps))


if __name__ == "__main__":
    main()
