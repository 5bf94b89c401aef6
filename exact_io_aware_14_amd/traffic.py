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
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_14_amd", "csrc")
OUT = os.path.join(ROOT, "profiles", "traffic.json")

COPY_BYTES = 512 << 20  # calibration copy: 512 MiB read + 512 MiB written
# HBM bytes versus sequence length: 16 heads, d = 128, causal, B*N = 16384 tokens
SWEEP_N = (1024, 2048, 4096, 8192, 16384)
SWEEP_OUT = os.path.join(ROOT, "profiles", "traffic_vs_n.md")
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


SWEEP_HEADER = """# HBM traffic against sequence length — 16 heads, d=128, bf16, causal, B*N = 16384 tokens

Commands, from the repository root on one MI355X (`TMPDIR=/tmp`):

    rocprofv3 --pmc FETCH_SIZE -f csv -d {sweep}/fetch -o p -- python -u bench.py --sweep-run
    rocprofv3 --pmc WRITE_SIZE -f csv -d {sweep}/write -o p -- python -u bench.py --sweep-run
    python -m exact_io_aware_14_amd.traffic {dir} --sweep {sweep}

Counters scaled by the calibration of profiles/traffic.json.  FETCH_SIZE and WRITE_SIZE count
the L2's requests to the memory fabric, so K/V re-reads that miss the per-XCD 4 MB L2 but hit the
256 MB last-level cache count here too.  Algorithmic bytes: the tensors
each kernel must read and write once (forward Q, K, V, O; dK/dV pass Q, K, V, dO, dK, dV; dQ pass,
which forms D = dO . O itself, Q, K, V, dO, O, dQ), lse/D vectors left out.  A materialised score matrix would grow 16x from the
first row to the last; the tiled method's traffic stays linear in N ("FlashAttention and online
softmax", "HBM traffic").  From N = 1024 to 8192 the ratios stay within {lo:.2f}-{hi:.2f}x.  At
N = 16384 (B = 1) one head's K and V (8 MB together) alone exceed an XCD's 4 MB L2, and the
causal head groups of the forward and the dQ pass hold two heads: their K/V re-reads miss L2
({big}).  Source hashes (forward, dK/dV pass, dQ pass): {hash}.

"""


def _code_only(text: str) -> str:
    """Source text without comments and blank space: a comment-only edit leaves the
    kernels, and so their counters, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# Source files each kernel's code comes from (besides the shared device headers).
KERNEL_SOURCES = {
    "fwd_kernel": ["fa_fwd_bf16.hip"],
    "bwd_main_kernel": ["fa_bwd_bf16.hip"],
    "bwd_dq_kernel": ["fa_bwd_dq_bf16.hip"],
    "bwd_pre_kernel": ["fa_bwd.hip"],
    "splitkv_partial_kernel": ["fa_decode.hip"],
    "splitkv_merge_kernel": ["fa_decode.hip"],
}
SHARED_SOURCES = ["fa_device.h", "fa_launch.h"]


def source_hash(kernel: str | None = None) -> str:
    """Hash of the sources (comments stripped) a kernel is compiled from: its own file
    and the shared device headers; with no kernel named, of every source."""
    names = sorted(os.listdir(CSRC)) if kernel is None else KERNEL_SOURCES[kernel] + SHARED_SOURCES
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
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
    for (name, _), v in sorted(per.items(), key=lambda kv: int(kv[0][1])):  # dispatch order
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
            kern.setdefault(label, {"source_hash": source_hash(label)})
            kern[label][key] = sum(vals) / len(vals) * 1024.0 * scale
    for wl, kern in out.items():
        if wl == "calibration":
            continue
        for e in kern.values():
            if "fetch_bytes" in e and "write_bytes" in e:
                e["hbm_bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
    return out


def sweep(dirpath: str, f_scale: float, w_scale: float) -> str:
    """Markdown table of HBM bytes per launch against N for the `--sweep-run` passes
    (one forward and one backward per N, in SWEEP_N order)."""
    fetch = read_counter(os.path.join(dirpath, "fetch"), "FETCH_SIZE")
    write = read_counter(os.path.join(dirpath, "write"), "WRITE_SIZE")
    rows = ["| kernel | N | B | HBM MB | algorithmic MB | ratio |", "|---|---|---|---|---|---|"]
    d, H, e = 128, 16, 2
    for frag, label, tensors in (("fwd_bf16_kernel", "forward", 4), ("bwd_bf16_kernel", "dK/dV pass", 6),
                                 ("bwd_dq_bf16_kernel", "dQ pass", 6)):
        names = [n for n in fetch if frag in n and ("dq" in frag) == ("dq" in n)]
        if not names:
            continue
        fv, wv = fetch[names[0]], write.get(names[0], [])
        for i, n in enumerate(SWEEP_N):
            if i >= len(fv) or i >= len(wv):
                break
            B = 16384 // n
            hbm = (fv[i] * f_scale + wv[i] * w_scale) * 1024.0
            alg = tensors * B * H * n * d * e
            rows.append(f"| {label} | {n} | {B} | {hbm / 1e6:.1f} | {alg / 1e6:.1f} | {hbm / alg:.3f} |")
    return "\n".join(rows)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("dir", help="directory holding the fetch/ and write/ rocprofv3 runs")
    ap.add_argument("--workload", default="long_causal")
    ap.add_argument("--sweep", default=None, help="directory of the --sweep-run passes: writes " + SWEEP_OUT)
    args = ap.parse_args(argv)
    if args.sweep:
        with open(OUT) as f:
            cal = json.load(f)["calibration"]
        table = sweep(args.sweep, cal["fetch_scale"], cal["write_scale"])
        with open(SWEEP_OUT, "w") as f:
            hashes = ", ".join(f"`{source_hash(k)}`" for k in ("fwd_kernel", "bwd_main_kernel", "bwd_dq_kernel"))
            cells = [c for c in (r.split("|") for r in table.splitlines()) if c[2].strip().isdigit()]
            small = [float(c[6]) for c in cells if int(c[2]) < 16384]
            big = ", ".join(f"{c[1].strip()} {float(c[6]):.2f}x" for c in cells if int(c[2]) == 16384)
            f.write(SWEEP_HEADER.format(hash=hashes, dir=args.dir.rstrip("/"), sweep=args.sweep.rstrip("/"),
                                        lo=min(small), hi=max(small), big=big)
                    + table + "\n")
        print(table)
        return 0
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
