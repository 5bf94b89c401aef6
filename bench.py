#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one forward (fa_fwd) and one backward (fa_bwd: for bf16 the dQ pass with
the preprocess folded in, then the dK/dV pass) over the workload's batch, inputs
resident in HBM.  Default workload: the long causal layer B=4, H=32, N=4096,
d=128, bf16 (planted query row), with dO as the fourth seeded draw.  FLOPs
credited: forward 4*B*H*N^2*d halved for causal, backward 2.5x that.

Prints one JSON line.  ``value`` is forward+backward TFLOP/s over the timed
steps (wall clock between device synchronisations).  ``roofline`` covers the
kernel with the largest average duration, timed with HIP events on the stream it
runs on; its FLOPs are the method's matrix products that kernel performs
(forward: 2 per visible score; dK/dV pass: 4; dQ pass: 1, its dQ product -- its
two recomputed products are not credited), each 2*d FLOPs.  ``clock`` is the
shader clock and board power sampled while the same step runs back to back for
1.5 s after the timed steps.  ``configs``
gives every workload's rates against both peak figures (2500 and 2516.6 TFLOP/s).
``cpu_baseline`` times the CPU fp64 oracle on a bounded sample of the same
workload (whole heads).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd & fwd+bwd (bf16, N=4096 d=128) + % MFMA peak"
PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_ALT = 2516.6     # the same peak as 256 CUs x 4 SIMDs x 1024 FLOP/clk x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel's current sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from exact_io_aware_14_amd.traffic import source_hash

    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != source_hash(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(x, w, heads, outs):
    """Time the oracle (fwd + bwd, fp64, naive) on whole heads of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from exact_io_aware_14_amd.accounting import fwd_flops
    from exact_io_aware_14_amd.inputs import to_f64
    from oracle import attention_bwd, attention_fwd

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t = 0.0
    backward = len(outs) == 5
    worst = {"O": 0.0, "lse": 0.0} | ({"dQ": 0.0, "dK": 0.0, "dV": 0.0} if backward else {})
    outs = [z.float().cpu().double().numpy() for z in outs]
    for (b, h) in heads:
        sl = lambda a: to_f64(a[b:b + 1, h:h + 1])
        Q, K, V = sl(x["q"]), sl(x["k"]), sl(x["v"])
        t0 = time.perf_counter()
        refs = list(attention_fwd(Q, K, V, w.scale, w.causal))
        if backward:
            refs += list(attention_bwd(Q, K, V, sl(x["do"]), w.scale, w.causal))
        t += time.perf_counter() - t0
        for (n, G, R) in zip(worst, outs, refs):
            err = float(np.abs(G[b:b + 1, h:h + 1] - R).max())
            if n not in ("O", "lse"):  # gradients: relative to the max-norm
                err /= float(np.abs(R).max())
            worst[n] = max(worst[n], err)
    credited = (3.5 if backward else 1.0) * fwd_flops(1, 1, w.N, w.d, w.causal) * len(heads)
    naive = (3.5 if backward else 1.0) * fwd_flops(1, 1, w.N, w.d, False) * len(heads)  # full N^2
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": credited / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "naive_flop_tflops": naive / t / 1e12,
        "cpu_model": cpu,
        "sample": f"{'fwd+bwd' if backward else 'fwd'} of {len(heads)} whole heads (b,h) in {heads[:3]}"
                  f"{'...' if len(heads) > 3 else ''} of the workload, "
                  f"N={w.N}, d={w.d}, fp64 numpy; credited FLOPs as for the GPU; {t:.1f} s",
        "seconds": t,
    }, {(n + ("_maxabs" if n in ("O", "lse") else "_rel")): e for n, e in worst.items()} | {"heads": len(heads)}


def decode_measure(dev, steps: int, warmup: int, cpu: bool):
    """Split-KV decoding on its workload: HIP-event time of the partial pass and of
    whole steps (the merge is their difference), HBM roofline of the partial pass, and
    the oracle timed beside it."""
    import numpy as np
    import torch

    from exact_io_aware_14_amd import fa
    from exact_io_aware_14_amd.accounting import splitkv_bytes
    from exact_io_aware_14_amd.inputs import DECODE_WORKLOADS, make_decode_inputs, to_f64

    w = DECODE_WORKLOADS["decode_long"]
    x = make_decode_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    S = w.splits
    op = torch.empty((S, w.B, w.H, w.Nq, w.d), dtype=torch.float32, device=dev)
    lp = torch.empty((S, w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    calls = [lambda: fa.fwd_partial(q, k, v, S, w.scale, w.causal, o_part=op, lse_part=lp),
             lambda: fa.merge(op, lp, q.dtype, out=o, lse=lse)]
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    # Back-to-back launches between one pair of events, so that the host-side cost of
    # each call (comparable to the merge's few microseconds) overlaps the GPU work
    # instead of showing up as idle time inside the timed region: first the partial
    # pass alone, then whole steps (partial + merge).
    def batch(fns):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            for f in fns:
                f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps
    part_us = batch(calls[:1])
    t0 = time.perf_counter()
    step_us = batch(calls)
    wall_us = (time.perf_counter() - t0) * 1e6 / steps
    merge_us = max(step_us - part_us, 0.0)
    b = splitkv_bytes(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, S)
    achieved = b["partial"] / (part_us * 1e-6) / 1e9
    rec = {
        "workload": {"name": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                     "causal": w.causal, "dtype": w.dtype, "splits": S},
        "partial_us": round(part_us, 2), "merge_us": round(merge_us, 2),
        "step_us_wall": round(wall_us, 2),
        "cache_GBps": round((b["partial"] + b["merge"]) / ((part_us + merge_us) * 1e-6) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "splitkv_partial_kernel", "achieved": round(achieved, 1),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(achieved / 8000.0, 4),
                     "traffic": measured_traffic("splitkv_partial_kernel", w.name)},
    }
    if cpu:
        from threadpoolctl import threadpool_info

        from oracle import attention_fwd_rect

        Q, K, V = (to_f64(x[n]) for n in ("q", "k", "v"))
        t1 = time.perf_counter()
        O_ref, lse_ref = attention_fwd_rect(Q, K, V, w.scale, w.causal)
        t = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        rec["cpu_baseline"] = {"value": round(b["partial"] / t / 1e9, 3), "unit": "GB/s of cache",
                               "cores": threads, "kind": "oracle",
                               "sample": f"the whole workload (all {w.B * w.H} heads), fp64 numpy, {t:.2f} s"}
        rec["parity_sample"] = {
            "O_maxabs": float(np.abs(o.float().cpu().numpy() - O_ref).max()),
            "lse_maxabs": float(np.abs(lse.cpu().numpy() - lse_ref).max())}
    return rec


def _timed(calls, steps: int, warmup: int):
    """Average HIP-event time (ms) of each callable, run in sequence per step."""
    import torch

    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for e in evs:
        for i, c in enumerate(calls):
            e[i].record()
            c()
        e[len(calls)].record()
    torch.cuda.synchronize()
    return [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(len(calls))]


KERNEL_NAMES = {"fwd": "fwd_kernel", "bwd_main": "bwd_main_kernel", "bwd_dq_pre": "bwd_dq_kernel",
                "bwd_dq": "bwd_dq_kernel", "bwd_preprocess": "bwd_pre_kernel"}


def _roofline(kernels: dict, workload: str) -> dict:
    """MFMA roofline of the longest kernel: kernels = {name: (ms, credited FLOPs)}."""
    dom = max(kernels, key=lambda n: kernels[n][0])
    ms, flops = kernels[dom]
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": KERNEL_NAMES[dom], "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": measured_traffic(KERNEL_NAMES[dom], workload)}


def _pct(tflops: float) -> dict:
    return {"tflops": round(tflops, 1), "pct_of_2500": round(100 * tflops / PEAK_TFLOPS, 2),
            "pct_of_2516.6": round(100 * tflops / PEAK_ALT, 2)}


def configs_measure(dev, steps: int, warmup: int, headline_name: str, headline: dict, cpu: bool) -> dict:
    """Every workload of the input recipe at full size: forward (and backward where the
    workload has one) time, TFLOP/s against both peak figures, the clock sampled while it
    ran and, with the CPU leg on, the errors of its last head against the oracle.  The
    headline layer's line comes from the main measurement."""
    import torch

    from exact_io_aware_14_amd import fa
    from exact_io_aware_14_amd.accounting import bwd_flops, fwd_flops
    from exact_io_aware_14_amd.inputs import WORKLOADS, make_inputs
    from exact_io_aware_14_amd.telemetry import soak

    out = {}
    for name, w in WORKLOADS.items():
        if name == headline_name:
            out[name] = headline
            continue
        x = make_inputs(w, with_do=True)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = fa.fwd(q, k, v, w.scale, w.causal)
        ws = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
        grads = tuple(torch.empty_like(q) for _ in range(3))
        calls = [lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)]
        if w.backward:
            calls.append(lambda: fa.bwd(q, k, v, o, do, lse, w.scale, w.causal, workspace=ws, grads=grads))
        par = None
        if cpu:  # the last head of the workload against the oracle
            for c in calls:
                c()
            torch.cuda.synchronize()
            _, par = cpu_baseline(x, w, [(w.B - 1, w.H - 1)], (o, lse) + (grads if w.backward else ()))
        if w.dtype != "bf16":  # the fp32 tiny case is a parity case, not a rate
            out[name] = {"workload": {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                                      "dtype": w.dtype}, "parity_sample": par}
            continue
        times = _timed(calls, steps, warmup)

        def one_step():
            for c in calls:
                c()
        clock = soak(one_step, 1.0, torch.cuda.synchronize)
        ff, bf = fwd_flops(w.B, w.H, w.N, w.d, w.causal), bwd_flops(w.B, w.H, w.N, w.d, w.causal)
        rec = {"workload": {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal},
               "fwd_ms": round(times[0], 4), "fwd": _pct(ff / times[0] / 1e9)}
        if w.backward:
            rec["bwd_ms"] = round(times[1], 4)
            rec["bwd"] = _pct(bf / times[1] / 1e9)
            rec["fwd_bwd"] = _pct((ff + bf) / (times[0] + times[1]) / 1e9)
        rec["clock"] = clock
        if par is not None:
            rec["parity_sample"] = par
        out[name] = rec
        del x, q, k, v, do, o, lse, ws, grads
    return out


def ex_measure(dev, steps: int, warmup: int, cpu: bool):
    """Sliding window (window_long) and variable-length batch (varlen_mix): fwd and bwd
    time, credited TFLOP/s over the visible pairs, and the same data without the
    feature (plain causal; zero-padded dense batch) timed beside it."""
    import numpy as np
    import torch

    from exact_io_aware_14_amd import fa
    from exact_io_aware_14_amd.accounting import varlen_pairs, window_pairs
    from exact_io_aware_14_amd.inputs import (VARLEN_WORKLOADS, WINDOW_WORKLOADS, make_inputs,
                                              make_varlen_inputs, to_f64)

    out = {}
    # --- sliding window ----------------------------------------------------------
    w, W = WINDOW_WORKLOADS["window_long"]
    x = make_inputs(w)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd_ex(q, k, v, w.scale, True, W)
    ws = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    t_f, t_dq, t_main = _timed([lambda: fa.fwd_ex(q, k, v, w.scale, True, W, out=o, lse=lse),
                                lambda: fa.bwd_ex(q, k, v, o, do, lse, w.scale, True, W, workspace=ws,
                                                  grads=grads, launches=1),
                                lambda: fa.bwd_ex(q, k, v, o, do, lse, w.scale, True, W, workspace=ws,
                                                  grads=grads, launches=2)],
                               steps, warmup)
    t_b = t_dq + t_main
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    c_f, c_b = _timed([lambda: fa.fwd(q, k, v, w.scale, True, out=o2, lse=lse2),
                       lambda: fa.bwd(q, k, v, o2, do, lse2, w.scale, True, workspace=ws, grads=grads)],
                      steps, warmup)
    ff = 4.0 * w.d * w.B * w.H * window_pairs(w.N, W)
    rec = {"workload": {"name": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "window": W,
                        "dtype": w.dtype},
           "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
           "fwd_tflops": round(ff / t_f / 1e9, 1), "bwd_tflops": round(2.5 * ff / t_b / 1e9, 1),
           "causal_without_window_ms": {"fwd": round(c_f, 4), "bwd": round(c_b, 4)},
           "speedup_vs_causal": round((c_f + c_b) / (t_f + t_b), 3),
           "visible_pair_ratio": round(window_pairs(w.N, 0) / window_pairs(w.N, W), 3),
           "kernel_ms": {"fwd": round(t_f, 4), "bwd_dq_pre": round(t_dq, 4), "bwd_main": round(t_main, 4)},
           "roofline": _roofline({"fwd": (t_f, ff), "bwd_dq_pre": (t_dq, 0.5 * ff), "bwd_main": (t_main, 2.0 * ff)},
                                 w.name)}
    if cpu:
        from oracle import attention_bwd, attention_fwd
        from oracle.varlen import window_mask

        sl = lambda t: to_f64(t[:, :1])
        Q, K, V, dO = (sl(x[n]) for n in ("q", "k", "v", "do"))
        t1 = time.perf_counter()
        m = window_mask(w.N, W)
        O_ref, _ = attention_fwd(Q, K, V, w.scale, True, mask=m)
        attention_bwd(Q, K, V, dO, w.scale, True, mask=m)
        t = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": round(3.5 * ff / (w.B * w.H) / t / 1e12, 5), "unit": "TFLOP/s",
                               "kind": "oracle", "sample": f"fwd+bwd of head (0,0), {t:.1f} s"}
        rec["parity_sample"] = {"O_maxabs_head0": float(np.abs(o[:, :1].float().cpu().numpy() - O_ref).max())}
    out["window_long"] = rec

    # --- variable-length batch ---------------------------------------------------
    vw = VARLEN_WORKLOADS["varlen_mix"]
    xv = make_varlen_inputs(vw)
    cu, nmax = xv["cu"].to(dev), xv["max_len"]
    lens = np.diff(xv["cu"].numpy())
    q, k, v, do = (xv[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd_ex(q, k, v, vw.scale, vw.causal, cu_seqlens=cu, max_seqlen=nmax)
    ws = torch.empty(fa.workspace_bytes(len(lens), vw.H, nmax, vw.d, q.dtype), dtype=torch.uint8, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    bx = lambda m: fa.bwd_ex(q, k, v, o, do, lse, vw.scale, vw.causal, cu_seqlens=cu, max_seqlen=nmax,
                             workspace=ws, grads=grads, validate=False, launches=m)
    t_f, t_dq, t_main = _timed([lambda: fa.fwd_ex(q, k, v, vw.scale, vw.causal, cu_seqlens=cu,
                                                  max_seqlen=nmax, out=o, lse=lse, validate=False),
                                lambda: bx(1), lambda: bx(2)], steps, warmup)
    t_b = t_dq + t_main
    # the same sequences zero-padded to the longest one, as a dense [B, H, max, d] batch
    B = len(lens)
    pad = lambda t: torch.zeros((B, vw.H, nmax, vw.d), dtype=t.dtype, device=dev)
    qp, kp, vp, dop = pad(q), pad(k), pad(v), pad(do)
    cuh = xv["cu"].numpy()
    for b in range(B):
        for src, dst in ((q, qp), (k, kp), (v, vp), (do, dop)):
            dst[b, :, :lens[b]] = src[:, cuh[b]:cuh[b + 1]]
    op, lsp = fa.fwd(qp, kp, vp, vw.scale, vw.causal)
    wsp = torch.empty(fa.workspace_bytes(B, vw.H, nmax, vw.d, q.dtype), dtype=torch.uint8, device=dev)
    gp = tuple(torch.empty_like(qp) for _ in range(3))
    p_f, p_b = _timed([lambda: fa.fwd(qp, kp, vp, vw.scale, vw.causal, out=op, lse=lsp),
                       lambda: fa.bwd(qp, kp, vp, op, dop, lsp, vw.scale, vw.causal, workspace=wsp, grads=gp)],
                      steps, warmup)
    ff = 4.0 * vw.d * vw.H * varlen_pairs(lens, vw.causal)
    rec = {"workload": {"name": vw.name, "sequences": B, "lengths": [int(n) for n in lens],
                        "total": int(lens.sum()), "max_len": nmax, "H": vw.H, "d": vw.d,
                        "causal": vw.causal, "dtype": vw.dtype},
           "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
           "fwd_tflops": round(ff / t_f / 1e9, 1), "bwd_tflops": round(2.5 * ff / t_b / 1e9, 1),
           "padded_dense_ms": {"fwd": round(p_f, 4), "bwd": round(p_b, 4)},
           "speedup_vs_padded": round((p_f + p_b) / (t_f + t_b), 3),
           "kernel_ms": {"fwd": round(t_f, 4), "bwd_dq_pre": round(t_dq, 4), "bwd_main": round(t_main, 4)},
           "roofline": _roofline({"fwd": (t_f, ff), "bwd_dq_pre": (t_dq, 0.5 * ff), "bwd_main": (t_main, 2.0 * ff)},
                                 vw.name)}
    if cpu:
        from oracle.varlen import varlen_fwd

        sl = lambda t: to_f64(t[:1])
        t1 = time.perf_counter()
        O_ref, _ = varlen_fwd(sl(xv["q"]), sl(xv["k"]), sl(xv["v"]), cuh, vw.scale, vw.causal)
        t = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": round(ff / vw.H / t / 1e12, 5), "unit": "TFLOP/s", "kind": "oracle",
                               "sample": f"forward of head 0, all sequences, {t:.1f} s"}
        rec["parity_sample"] = {"O_maxabs_head0": float(np.abs(o[:1].float().cpu().numpy() - O_ref).max())}
    out["varlen_mix"] = rec
    return out


def secondary_measure(dev, steps: int, warmup: int):
    """The long layer without the causal mask (secondary headline), and a cold-cache
    variant of the two workloads whose inputs fit in the 256 MB last-level cache: a
    1 GiB scratch buffer is written between calls, so every call reads HBM."""
    import torch

    from exact_io_aware_14_amd import fa
    from exact_io_aware_14_amd.accounting import bwd_flops, fwd_flops
    from exact_io_aware_14_amd.inputs import WORKLOADS, make_inputs

    out = {}
    w = WORKLOADS["long_causal"].with_(name="long_noncausal", causal=False, planted=None)
    x = make_inputs(w, with_do=True)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, w.scale, False)
    ws = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    t_f, t_b = _timed([lambda: fa.fwd(q, k, v, w.scale, False, out=o, lse=lse),
                       lambda: fa.bwd(q, k, v, o, do, lse, w.scale, False, workspace=ws, grads=grads)],
                      steps, warmup)
    ff, bf = fwd_flops(w.B, w.H, w.N, w.d, False), bwd_flops(w.B, w.H, w.N, w.d, False)
    out["long_noncausal"] = {"workload": {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": False},
                             "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
                             "fwd_tflops": round(ff / t_f / 1e9, 1), "bwd_tflops": round(bf / t_b / 1e9, 1),
                             "fwd_bwd_tflops": round((ff + bf) / (t_f + t_b) / 1e9, 1)}
    del q, k, v, do, o, lse, ws, grads
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for name in ("gpt2m_fwd", "train_step"):
        w = WORKLOADS[name]
        x = make_inputs(w, with_do=True)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = fa.fwd(q, k, v, w.scale, w.causal)
        ws = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
        grads = tuple(torch.empty_like(q) for _ in range(3))
        fw = lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        bw = lambda: fa.bwd(q, k, v, o, do, lse, w.scale, w.causal, workspace=ws, grads=grads)
        warm = _timed([fw, bw], steps, warmup)
        cold = _timed([lambda: scratch.fill_(1), fw, lambda: scratch.fill_(2), bw], steps, warmup)
        ff, bf = fwd_flops(w.B, w.H, w.N, w.d, w.causal), bwd_flops(w.B, w.H, w.N, w.d, w.causal)
        out[name] = {"workload": {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal},
                     "warm": {"fwd_ms": round(warm[0], 4), "bwd_ms": round(warm[1], 4),
                              "fwd_tflops": round(ff / warm[0] / 1e9, 1), "bwd_tflops": round(bf / warm[1] / 1e9, 1)},
                     "cold": {"fwd_ms": round(cold[1], 4), "bwd_ms": round(cold[3], 4),
                              "fwd_tflops": round(ff / cold[1] / 1e9, 1), "bwd_tflops": round(bf / cold[3] / 1e9, 1)}}
    return out


def traffic_run_ex(dev, name: str) -> int:
    """For rocprofv3 counter passes on the windowed or variable-length workload: the
    calibration copy, then its forward and backward twice (warm-up, counted)."""
    import torch

    from exact_io_aware_14_amd import fa
    from exact_io_aware_14_amd.inputs import (VARLEN_WORKLOADS, WINDOW_WORKLOADS, make_inputs,
                                              make_varlen_inputs)
    from exact_io_aware_14_amd.traffic import COPY_BYTES

    if name in WINDOW_WORKLOADS:
        w, W = WINDOW_WORKLOADS[name]
        x = make_inputs(w)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
        args = dict(scale=w.scale, causal=True, window=W)
    elif name in VARLEN_WORKLOADS:
        vw = VARLEN_WORKLOADS[name]
        xv = make_varlen_inputs(vw)
        q, k, v, do = (xv[n].to(dev) for n in ("q", "k", "v", "do"))
        args = dict(scale=vw.scale, causal=vw.causal, cu_seqlens=xv["cu"].to(dev), max_seqlen=xv["max_len"])
    else:
        print(f"unknown workload {name}", file=sys.stderr)
        return 2

    def run():
        o, lse = fa.fwd_ex(q, k, v, **args)
        fa.bwd_ex(q, k, v, o, do, lse, **args)

    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    run()
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": name, "copy_bytes": COPY_BYTES}), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_causal")
    ap.add_argument("--cpu-heads", type=int, default=64, help="heads in the CPU oracle sample (0 = skip)")
    ap.add_argument("--no-next", action="store_true", help="skip the NEXT-row and secondary measurements")
    ap.add_argument("--sweep-run", action="store_true",
                    help="for rocprofv3 counter passes: fwd and bwd once at N = 1024..16384, B*N = 16384")
    ap.add_argument("--traffic-run", action="store_true",
                    help="for rocprofv3 counter passes: a calibration copy, then each kernel once")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the attention hot path here has no multi-GPU "
              f"path (asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        return 2

    import torch

    from exact_io_aware_14_amd import fa
    from exact_io_aware_14_amd.accounting import bwd_flops, fwd_flops
    from exact_io_aware_14_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    fa.lib()
    dev = torch.device("cuda:0")
    if args.traffic_run and args.workload not in WORKLOADS:
        return traffic_run_ex(dev, args.workload)
    w = WORKLOADS[args.workload]
    x = make_inputs(w, with_do=True)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
    stages = fa.bwd_stages(q, k, v, o, do, lse, w.scale, w.causal, ws, grads, fused=True)
    names = ["fwd"] + (["bwd_dq_pre", "bwd_main"] if len(stages) == 2 else
                       ["bwd_preprocess", "bwd_main", "bwd_dq"])
    calls = [lambda: fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)] + stages

    def step(evs=None):
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i].record()
            c()
        if evs is not None:
            evs[len(calls)].record()

    if args.sweep_run:
        from exact_io_aware_14_amd.traffic import SWEEP_N

        for n in SWEEP_N:
            ws_ = WORKLOADS["long_context"].with_(name=f"sweep{n}", B=16384 // n, N=n)
            xs = make_inputs(ws_, with_do=True)
            qs, ks, vs, dos = (xs[m].to(dev) for m in ("q", "k", "v", "do"))
            os_, ls_ = fa.fwd(qs, ks, vs, ws_.scale, True)
            fa.bwd(qs, ks, vs, os_, dos, ls_, ws_.scale, True)
            torch.cuda.synchronize()
            del qs, ks, vs, dos, os_, ls_
        print(json.dumps({"sweep_run": list(SWEEP_N)}), flush=True)
        return 0

    if args.traffic_run:
        from exact_io_aware_14_amd.traffic import COPY_BYTES

        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        step()  # warm-up
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # calibration: reads and writes COPY_BYTES each
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        decode_measure(dev, 1, 1, False)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_run": w.name, "copy_bytes": COPY_BYTES}), flush=True)
        return 0

    from exact_io_aware_14_amd.telemetry import soak

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the clock and power of the same step held for ~1.5 s (the metrics refresh ~1/s)
    clock = soak(step, 1.5, torch.cuda.synchronize)
    ms_step = (t1 - t0) * 1e3 / args.steps
    per = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i, n in enumerate(names)}
    samples = {n: sorted(e[i].elapsed_time(e[i + 1]) for e in evs) for i, n in enumerate(names)}
    med = {n: v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
           for n, v in samples.items()}

    ff = fwd_flops(w.B, w.H, w.N, w.d, w.causal)
    bf = bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    bwd_ms = sum(per[n] for n in names[1:])
    value = (ff + bf) / (ms_step * 1e-3) / 1e12
    fwd_t = ff / (per["fwd"] * 1e-3) / 1e12
    bwd_t = bf / (bwd_ms * 1e-3) / 1e12
    # the method's products each kernel performs (2*d FLOPs per visible score each):
    # forward 2, dK/dV pass 4, dQ pass 1 (its recomputed S and dP are not credited)
    kflops = {"fwd": ff, "bwd_main": 2.0 * ff, "bwd_dq_pre": 0.5 * ff, "bwd_dq": 0.5 * ff, "bwd_preprocess": 0.0}
    roof = _roofline({n: (per[n], kflops[n]) for n in names}, w.name)
    # executed matrix FLOPs (dQ pass: 3 products), for comparison with the MFMA counters
    xflops = {"fwd": ff, "bwd_main": 2.0 * ff, "bwd_dq_pre": 1.5 * ff, "bwd_dq": 1.5 * ff, "bwd_preprocess": 0.0}

    props = torch.cuda.get_device_properties(dev)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "planted_row": list(w.planted) if w.planted else None,
                   "step": "fa_fwd + fa_bwd"},
        "fwd_tflops": round(fwd_t, 2),
        "fwd_pct_peak": round(100 * fwd_t / PEAK_TFLOPS, 2),
        "bwd_tflops": round(bwd_t, 2),
        "bwd_pct_peak": round(100 * bwd_t / PEAK_TFLOPS, 2),
        "fwd_bwd_pct_peak": round(100 * value / PEAK_TFLOPS, 2),
        "pct_of_2516.6": {"fwd": round(100 * fwd_t / PEAK_ALT, 2), "bwd": round(100 * bwd_t / PEAK_ALT, 2),
                          "fwd_bwd": round(100 * value / PEAK_ALT, 2)},
        "kernel_ms": {n: round(m, 4) for n, m in per.items()},
        "kernel_ms_median": {n: round(m, 4) for n, m in med.items()},
        "kernel_ms_min": {n: round(v[0], 4) for n, v in samples.items()},
        "kernel_executed_tflops": {n: round(xflops[n] / (per[n] * 1e-3) / 1e12, 1) for n in names},
        "roofline": roof,
        "clock": clock,
        "device": props.name,
    }
    headline = {"workload": {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal},
                "fwd_ms": round(per["fwd"], 4), "fwd": _pct(fwd_t), "bwd_ms": round(bwd_ms, 4),
                "bwd": _pct(bwd_t), "fwd_bwd": _pct((ff + bf) / ((per["fwd"] + bwd_ms) * 1e-3) / 1e12),
                "clock": rec["clock"]}
    if args.cpu_heads > 0:
        heads = [(i // w.H, i % w.H) for i in range(min(args.cpu_heads, w.B * w.H))]
        cb, par = cpu_baseline(x, w, heads, (o, lse) + grads)
        rec["cpu_baseline"] = cb
        rec["parity_sample"] = par
        headline["parity_sample"] = par
    else:
        rec["cpu_baseline"] = None
    if not args.no_next:
        rec["next_rows"] = {"splitkv_decode": decode_measure(dev, args.steps, args.warmup, args.cpu_heads > 0)}
        rec["next_rows"].update(ex_measure(dev, min(args.steps, 10), min(args.warmup, 3), args.cpu_heads > 0))
        rec["secondary"] = secondary_measure(dev, min(args.steps, 10), min(args.warmup, 3))
        rec["configs"] = configs_measure(dev, min(args.steps, 10), min(args.warmup, 3), w.name, headline,
                                         args.cpu_heads > 0)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
