"""HBM traffic per kernel launch from rocprofv3 counter runs.

Two commands, each a separate rocprofv3 pass (one counter block per pass):

    rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/fetch -o p -- python bench.py --traffic-run
    rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/write -o p -- python bench.py --traffic-run
    python -m exact_io_aware_14_amd.traffic <dir> [--workload long_causal]

``bench.py --traffic-run`` launches, once each after a warm-up: a plain device
copy of a known size (the calibration kernel), the forward, the three backward
stages, and the two split-KV decoding passes on the decoding workload.  FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch; the copy of
C bytes must read C and write C bytes, so each counter is scaled by C / (what it
reads for the copy).  The result, with the hash of the kernel sources it was taken
on, goes to profiles/traffic.json, which bench.py reads (and ignores once the
sources change).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_14_amd", "csrc")
OUT = os.path.join(ROOT, "profiles", "traffic.json")

COPY_BYTES = 512 << 20  # calibration copy: 512 MiB read + 512 MiB written
# kernel-name fragments -> (workload the traffic run launches it on, name used in
# bench.py's roofline)
KERNELS = {
    "fwd_bf16_kernel": (None, "fwd_kernel"),
    "bwd_bf16_kernel": (None, "bwd_main_kernel"),
    "bwd_dq_bf16_kernel": (None, "bwd_dq_kernel"),
    "bwd_pre_kernel": (None, "bwd_pre_kernel"),
    "splitkv_partial_kernel": ("decode_long", "splitkv_partial_kernel"),
    "splitkv_merge_kernel": ("decode_long", "splitkv_merge_kernel"),
}


def source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_counter(dirpath: str, counter: str) -> dict:
    """{kernel name: [KiB per dispatch, ...]} for one counter from a rocprofv3 csv dir."""
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {dirpath}")
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def classify(name: str):
    """(workload or None for the main one, label) of a kernel name, or None."""
    for frag, wl in KERNELS.items():
        if frag in name:
            return wl
    return None


def summarize(dirpath: str, workload: str) -> dict:
    fetch = read_counter(os.path.join(dirpath, "fetch"), "FETCH_SIZE")
    write = read_counter(os.path.join(dirpath, "write"), "WRITE_SIZE")
    # the calibration copy is the only elementwise copy kernel in the run
    def copy_kib(d):
        vals = [v for n, vs in d.items() if "copy" in n.lower() or "elementwise" in n.lower() for v in vs]
        if not vals:
            raise RuntimeError("calibration copy kernel not found in the counter run")
        return max(vals)
    f_scale = COPY_BYTES / (copy_kib(fetch) * 1024.0)
    w_scale = COPY_BYTES / (copy_kib(write) * 1024.0)
    res = {"source_hash": source_hash(), "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale}
    out = {"calibration": res}
    for d, scale, key in ((fetch, f_scale, "fetch_bytes"), (write, w_scale, "write_bytes")):
        for name, vals in d.items():
            c = classify(name)
            if c is None:
                continue
            wl, label = c
            kern = out.setdefault(wl or workload, {})
            kern.setdefault(label, {"source_hash": res["source_hash"]})
            kern[label][key] = sum(vals) / len(vals) * 1024.0 * scale
    for wl, kern in out.items():
        if wl == "calibration":
            continue
        for e in kern.values():
            if "fetch_bytes" in e and "write_bytes" in e:
                e["hbm_bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("dir", help="directory holding the fetch/ and write/ rocprofv3 runs")
    ap.add_argument("--workload", default="long_causal")
    args = ap.parse_args(argv)
    s = summarize(args.dir, args.workload)
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    old = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            old = json.load(f)
    old.update(s)
    with open(OUT, "w") as f:
        json.dump(old, f, indent=1, sort_keys=True)
    print(json.dumps(s, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
