"""Per-kernel hardware counters from rocprofv3 ``--pmc`` passes, summarised as the
figures that say which unit bounds each kernel: MFMA-busy, VALU-busy and LDS
activity against elapsed cycles, instruction mixes, and the shader clock.

Each pass is a separate rocprofv3 run (a pass holds at most 8 SQ and 2 GRBM
counters on gfx950), over ``bench.py --traffic-run`` which launches every kernel
once after a warm-up step::

    rocprofv3 --pmc <PASSES["busy"]> -f csv -d <dir>/busy -o p -- python -u bench.py --traffic-run [--workload W]
    rocprofv3 --pmc <PASSES["mix"]>  -f csv -d <dir>/mix  -o p -- python -u bench.py --traffic-run [--workload W]
    rocprofv3 --pmc <PASSES["stall"]> -f csv -d <dir>/stall -o p -- python -u bench.py --traffic-run [--workload W]
    rocprofv3 --kernel-trace --stats -d <dir>/trace -o p -- python -u bench.py --traffic-run [--workload W]
    python -m exact_io_aware_14_amd.counters <dir> --workload W [--out profiles/counters_W.md]

Definitions (counter semantics from the rocprofiler counter definitions for gfx950,
checked against the runs):
* GRBM_GUI_ACTIVE counts shader-clock cycles while the GPU is busy; the csv holds its
  sum over the 8 XCDs, so elapsed cycles = GRBM_GUI_ACTIVE / 8, and elapsed cycles /
  the dispatch's duration is the mean shader clock.
* SQ_VALU_MFMA_BUSY_CYCLES, summed over the 1024 SIMDs, adds 32 cycles per
  32x32x16 bf16 MFMA (it equals 32 x SQ_INSTS_MFMA in these kernels); MFMA-busy % =
  that / (elapsed cycles x 1024), the ``MfmaUtil`` derived metric.  MFMA-busy x
  clock / 2.4 GHz is the executed matrix rate as a fraction of the 2.5 PFLOP/s peak,
  which SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP / duration gives independently.
* SQ_ACTIVE_INST_VALU and SQ_ACTIVE_INST_LDS are quad-cycles summed over the waves
  of a CU; 100 x value / (256 CUs x elapsed cycles) is the ``VALUBusy`` metric: the
  share of cycles a SIMD spends issuing vector (resp. LDS) instructions.
* SQ_LDS_IDX_ACTIVE / (256 x elapsed cycles): the share of cycles each CU's LDS is busy.
* Where a wave's cycles go (the optional stall pass), as shares of SQ_WAVE_CYCLES:
  SQ_WAIT_ANY (waiting on a counter or the barrier), SQ_WAIT_INST_ANY (ready but waiting
  to issue: a dependency or a busy unit) and SQ_ACTIVE_INST_ANY (issuing); and
  SQ_VALU_MFMA_COEXEC_CYCLES over the vector-busy cycles 4 x SQ_ACTIVE_INST_VALU: the
  share of vector work that runs while the wave's MFMA work does.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N_CU, N_SIMD, N_XCD = 256, 1024, 8
PEAK_BF16 = 2500.0e12  # dense bf16 MFMA FLOP/s, published
REF_CLOCK = 2.4e9      # clock the published peak is quoted at

PASSES = {
    "busy": ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAVES",
             "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"],
    "mix": ["GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
            "SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
            "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY"],
    "stall": ["GRBM_GUI_ACTIVE", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
              "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU2", "SQ_INSTS_VMEM_RD",
              "SQ_ACTIVE_INST_SCA", "SQ_WAVE_CYCLES"],
}

# kernel-name fragments -> label (the first fragment found in a name wins)
KERNELS = [("bwd_dq_bf16_kernel", "dQ pass"), ("bwd_bf16_kernel", "dK/dV pass"),
           ("fwd_bf16_kernel", "forward"), ("bwd_pre_kernel", "bwd preprocess"),
           ("splitkv_partial_kernel", "split-KV partial"), ("splitkv_merge_kernel", "split-KV merge")]


def label(name: str):
    for frag, lab in KERNELS:
        if frag in name:
            return lab
    return None


def read_pass(dirpath: str) -> dict:
    """{label: {counter: mean value per dispatch}} of one rocprofv3 csv directory."""
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {dirpath}")
    per = {}  # (label, dispatch) -> {counter: value}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                lab = label(row["Kernel_Name"])
                if lab is None:
                    continue
                d = per.setdefault((lab, int(row["Dispatch_Id"])), {})
                c = row["Counter_Name"]
                d[c] = d.get(c, 0.0) + float(row["Counter_Value"])
    out = {}
    for (lab, _), vals in per.items():
        acc = out.setdefault(lab, {})
        for c, v in vals.items():
            acc.setdefault(c, []).append(v)
    return {lab: {c: sum(v) / len(v) for c, v in cs.items()} for lab, cs in out.items()}


def read_durations(dirpath: str) -> dict:
    """{label: mean kernel duration in seconds} from a rocprofv3 kernel trace."""
    files = glob.glob(os.path.join(dirpath, "**", "*kernel_trace.csv"), recursive=True)
    dur = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                lab = label(row["Kernel_Name"])
                if lab is None:
                    continue
                dur.setdefault(lab, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9)
    # the run launches each kernel after a warm-up launch: keep the later, warm ones
    return {lab: (sum(v[len(v) // 2:]) / len(v[len(v) // 2:])) for lab, v in dur.items()}


def _clock(dirpath: str) -> dict:
    """{label: mean shader clock in Hz} from the counter pass's own dispatch times."""
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    clk = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                lab = label(row["Kernel_Name"])
                if lab is None or row["Counter_Name"] != "GRBM_GUI_ACTIVE":
                    continue
                t = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
                clk.setdefault(lab, []).append(float(row["Counter_Value"]) / N_XCD / t)
    return {lab: sum(v) / len(v) for lab, v in clk.items()}


def summarize(dirpath: str, workload: str) -> str:
    busy = read_pass(os.path.join(dirpath, "busy"))
    mix = read_pass(os.path.join(dirpath, "mix"))
    clock = _clock(os.path.join(dirpath, "busy"))
    dur = read_durations(os.path.join(dirpath, "trace")) if os.path.isdir(os.path.join(dirpath, "trace")) else {}
    rows = ["| kernel | time µs (trace) | clock GHz | MFMA busy % | x clock/2.4 GHz | executed bf16 % of 2.5 PF (FLOP count / time) | "
            "VALU busy % | LDS-issue busy % | LDS unit busy % | LDS instr / MFMA | VALU instr / MFMA | exp / MFMA | "
            "bank-conflict % of LDS cycles |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for lab in [l for _, l in KERNELS]:
        if lab not in busy or busy[lab].get("SQ_INSTS_MFMA", 0.0) == 0.0:
            continue
        b, m = busy[lab], mix.get(lab, {})
        cyc = b["GRBM_GUI_ACTIVE"] / N_XCD
        cyc_m = m.get("GRBM_GUI_ACTIVE", b["GRBM_GUI_ACTIVE"]) / N_XCD
        t = dur.get(lab, float("nan"))
        f = clock.get(lab, float("nan"))
        mfma_busy = 100.0 * b["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        flops = b["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        frac = 100.0 * flops / t / PEAK_BF16
        valu = 100.0 * b["SQ_ACTIVE_INST_VALU"] / (N_CU * cyc)
        lds_issue = 100.0 * b["SQ_ACTIVE_INST_LDS"] / (N_CU * cyc)
        lds_unit = 100.0 * m.get("SQ_LDS_IDX_ACTIVE", float("nan")) / (N_CU * cyc_m)
        nm = b["SQ_INSTS_MFMA"]
        conflict = 100.0 * m.get("SQ_LDS_BANK_CONFLICT", float("nan")) / max(m.get("SQ_LDS_IDX_ACTIVE", 1.0), 1.0)
        rows.append(f"| {lab} | {t * 1e6:.1f} | {f / 1e9:.2f} | {mfma_busy:.1f} | {mfma_busy * f / REF_CLOCK:.1f} | "
                    f"{frac:.1f} | {valu:.1f} | {lds_issue:.1f} | {lds_unit:.1f} | "
                    f"{m.get('SQ_INSTS_LDS', float('nan')) / nm:.2f} | {m.get('SQ_INSTS_VALU', float('nan')) / nm:.2f} | "
                    f"{m.get('SQ_INSTS_VALU_TRANS_F32', float('nan')) / nm:.2f} | {conflict:.2f} |")
    stall_dir = os.path.join(dirpath, "stall")
    stall = read_pass(stall_dir) if os.path.isdir(stall_dir) else {}
    if stall:
        rows += ["", "Where the waves' cycles go (stall pass; shares of `SQ_WAVE_CYCLES`; the last column is",
                 "`SQ_VALU_MFMA_COEXEC_CYCLES` over the vector-busy cycles `4 x SQ_ACTIVE_INST_VALU`):", "",
                 "| kernel | waiting for anything | waiting to issue | issuing | VALU cycles that overlap MFMA work |",
                 "|---|---|---|---|---|"]
        for lab in [l for _, l in KERNELS]:
            if lab not in stall or lab not in busy or busy[lab].get("SQ_INSTS_MFMA", 0.0) == 0.0:
                continue
            s, b = stall[lab], busy[lab]
            wc = s["SQ_WAVE_CYCLES"]
            rows.append(f"| {lab} | {100 * s['SQ_WAIT_ANY'] / wc:.0f} % | {100 * s['SQ_WAIT_INST_ANY'] / wc:.0f} % | "
                        f"{100 * s['SQ_ACTIVE_INST_ANY'] / wc:.0f} % | "
                        f"{100 * s['SQ_VALU_MFMA_COEXEC_CYCLES'] / (4 * b['SQ_ACTIVE_INST_VALU']):.0f} % |")
    raw = ["", "Raw counters (mean per dispatch; GRBM_GUI_ACTIVE summed over the 8 XCDs):", "",
           "| kernel | counter | value |", "|---|---|---|"]
    for lab in [l for _, l in KERNELS]:
        for src in (busy, mix, stall):
            for c, v in sorted(src.get(lab, {}).items()):
                raw.append(f"| {lab} | {c} | {v:.6g} |")
    return "\n".join(rows + raw) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("dir", help="directory holding the busy/, mix/ and trace/ rocprofv3 runs")
    ap.add_argument("--workload", default="long_causal")
    ap.add_argument("--out", default=None, help="markdown file to write the table to")
    args = ap.parse_args(argv)
    text = summarize(args.dir, args.workload)
    print(text)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
