"""Build libfa.so (the HIP kernels + C ABI) for gfx950, in-tree.

    python -m exact_io_aware_14_amd.build [--verbose] [--save-temps DIR]

hipcc cross-compiles for gfx950 without a GPU.  Packed fp32 VALU ops are turned
off (-packed-fp32-ops) for every HIP source.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_bf16.hip", "fa_bwd.hip", "fa_bwd_bf16.hip", "fa_bwd_dq_bf16.hip", "fa_decode.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfa.so")


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            extra = []
            if save_temps:
                obj_dir = os.path.abspath(os.path.join(save_temps, src.replace(".hip", "")))
                os.makedirs(obj_dir, exist_ok=True)
                obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
                extra = ["-save-temps=obj", "-Rpass-analysis=kernel-resource-usage"]
            cmd = [cc, *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            out = (r.stdout + r.stderr)
            # hipcc's host pass does not know the gfx950 feature name: harmless
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{out}")
            if verbose and out.strip():
                print(out)
            return obj

        # one hipcc per source, run side by side (each is a separate process)
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None)
    args = ap.parse_args(argv)
    path = build(args.verbose, args.save_temps)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
