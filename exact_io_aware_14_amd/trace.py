"""Per-kernel durations from a rocprofv3 kernel trace (``--kernel-trace``), as the
markdown table the profiles quote.

    rocprofv3 --kernel-trace --stats -f csv -d <dir> -o p -- python -u bench.py --no-next --cpu-heads 0
    python -m exact_io_aware_14_amd.trace <dir> [--title TEXT]

Kernels are named by what they compute; the template arguments tell the head dim and
whether the general (windowed / variable-length) instantiation ran.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys

LABELS = [("bwd_dq_bf16_kernel", "dQ pass"), ("bwd_bf16_kernel", "dK/dV pass"), ("bwd_plan_kernel", "dK/dV plan"),
          ("fwd_bf16_kernel", "forward"),
          ("bwd_pre_kernel", "bwd preprocess"), ("splitkv_partial_kernel", "split-KV partial"),
          ("splitkv_merge_kernel", "split-KV merge")]


def label(name: str):
    for frag, lab in LABELS:
        if frag in name:
            m = re.search(frag + r"<([^>]*)>", name)
            return f"{lab} <{m.group(1)}>" if m else lab
    return None


def durations(dirpath: str) -> dict:
    files = glob.glob(os.path.join(dirpath, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {dirpath}")
    out = {}
    for f in files:
        with open(f) as fh:
            rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            lab = label(r["Kernel_Name"])
            if lab is not None:
                out.setdefault(lab, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def table(dirpath: str) -> str:
    d = durations(dirpath)
    lines = ["| kernel | calls | mean µs | median µs | min µs | max µs |", "|---|---|---|---|---|---|"]
    for lab in sorted(d):
        v = d[lab]
        lines.append(f"| {lab} | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} |")
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    args = ap.parse_args(argv)
    print(table(args.dir))
    return 0


if __name__ == "__main__":
    sys.exit(main())
