"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Small cases span several tiles and a ragged tail and are compared element by
element in full.  The five full-size workloads run at their real shapes with the
same launch configuration the benchmark times; every output of whole sampled
heads is compared (a head is the oracle's independent unit of work).
"""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_14_amd import fa
from exact_io_aware_14_amd.inputs import WORKLOADS, Workload, draw_f32, finish_inputs, make_inputs, to_f64
from oracle import attention_bwd, attention_fwd
from oracle.splitkv import attention_fwd_rect
from parity import check_fwd, check_grad, f64

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.lib()  # fail loudly if the native library is missing
    return torch.device("cuda:0")


def gpu_fwd(x, w, dev):
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))  # catches unwritten elements
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=dev)
    fa.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
    return q, k, v, o, lse


def gpu_bwd(q, k, v, o, lse, do, w, dev):
    nb = fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=dev)  # NaN garbage: must be cleared
    grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    return fa.bwd(q, k, v, o, do, lse, w.scale, w.causal, workspace=ws, grads=grads)


# N = 1 and 7: one partial tile; 90, 300 and 1000 give 3, 10 and 32 query tiles of 32 rows,
# so the backward's four-set tile rotation ends at every remainder (mod 4) it can have.
SMALL = [(1, 1, 1), (1, 1, 7), (1, 2, 90), (2, 3, 300), (1, 2, 1000)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dN%d" % s)
def test_small_fwd_bwd(dev, dtype, d, causal, shape):
    B, H, N = shape
    w = Workload("small", B, H, N, d, causal, dtype, True, seed=N + d)
    say(f"[small] {dtype} B={B} H={H} N={N} d={d} causal={causal}")
    x = make_inputs(w)
    q, k, v, o, lse = gpu_fwd(x, w, dev)
    Q, K, V, dO = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    O_ref, lse_ref = attention_fwd(Q, K, V, w.scale, causal)
    torch.cuda.synchronize()
    check_fwd(dtype, o, lse, O_ref, lse_ref, "fwd")
    do = x["do"].to(dev)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, do, w, dev)
    torch.cuda.synchronize()
    dQ, dK, dV = attention_bwd(Q, K, V, dO, w.scale, causal)
    for G, R, n in ((dq, dQ, "dQ"), (dk, dK, "dK"), (dv, dV, "dV")):
        check_grad(dtype, G, R, n, "bwd")


def _full(name):
    return WORKLOADS[name]


HEADS = {
    "tiny_fp32": [(0, 0)],
    "gpt2m_fwd": [(0, 0), (7, 15)],
    # 16 heads spread over the dispatch groups of two heads (b*H + h = 0, 9, 17, ... 127):
    # both members of a pair, first and last groups, every batch
    "long_causal": [(bh // 32, bh % 32) for bh in (0, 9, 17, 26, 34, 43, 51, 60, 68, 77, 85, 94,
                                                   102, 111, 119, 127)],
    "train_step": [(0, 0), (3, 15)],
    "long_context": [(0, 0), (0, 5), (0, 10), (0, 15)],
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(dev, name):
    """Full-size workload on the GPU; every output element of the sampled heads vs the oracle.
    long_causal also runs the backward (the fwd+bwd headline shape, dO = 4th draw)."""
    w = _full(name)
    backward = w.backward
    say(f"[workload] {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} {w.dtype} bwd={backward}")
    x = make_inputs(w, with_do=backward)
    q, k, v, o, lse = gpu_fwd(x, w, dev)
    if backward:
        dq, dk, dv = gpu_bwd(q, k, v, o, lse, x["do"].to(dev), w, dev)
    torch.cuda.synchronize()
    for (b, h) in HEADS[name]:
        sl = lambda t: to_f64(t[b:b + 1, h:h + 1])
        Q, K, V = sl(x["q"]), sl(x["k"]), sl(x["v"])
        say(f"  oracle head ({b},{h})")
        O_ref, lse_ref = attention_fwd(Q, K, V, w.scale, w.causal)
        check_fwd(w.dtype, o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], O_ref, lse_ref, f"{name}({b},{h})")
        if backward:
            dQ, dK, dV = attention_bwd(Q, K, V, sl(x["do"]), w.scale, w.causal)
            for G, R, n in ((dq, dQ, "dQ"), (dk, dK, "dK"), (dv, dV, "dV")):
                check_grad(w.dtype, G[b:b + 1, h:h + 1], R, n, f"{name}({b},{h})")
    # outputs of every head are finite and fully written
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    if backward:
        for G in (dq, dk, dv):
            assert torch.isfinite(G).all().item()


def test_planted_row_exercises_rescaling(dev):
    """The planted query row (scaled x30) has scores far beyond exp's fp32 range
    unless the running max is subtracted; its output still matches the oracle."""
    w = _full("long_causal").with_(B=1, H=1)
    say("[planted] long_causal head (0,0)")
    x = make_inputs(w, with_do=False)
    q, k, v, o, lse = gpu_fwd(x, w, dev)
    torch.cuda.synchronize()
    row = w.planted[2]
    Q, K, V = (to_f64(x[n]) for n in ("q", "k", "v"))
    S = w.scale * Q[0, 0, row] @ K[0, 0, :row + 1].T
    assert S.max() * math.log2(math.e) > 128  # 2^s would overflow fp32 without the max
    O_ref, lse_ref = attention_fwd(Q, K, V, w.scale, True)
    check_fwd("bf16", o[:, :, row:row + 1], lse[:, :, row:row + 1], O_ref[:, :, row:row + 1],
              lse_ref[:, :, row:row + 1], "planted")


# Planted rows of the long causal layer (query row x 30 before rounding): the default
# (0, 0, 2049), its neighbours across the 2048 tile boundary, the last row of the first
# and last heads, and rows of other heads.  On such a nearly one-hot row dS = P (dP - D)
# cancels two close numbers, and D = dO . O from the bf16 O is the largest error in dK.
PLANTED = [(0, 0, 2049), (0, 0, 2047), (0, 0, 2048), (0, 0, 4095), (3, 31, 4095), (2, 5, 1023),
           (0, 0, 63), (1, 9, 3000)]


@pytest.mark.timeout(900)
def test_planted_rows_full_size(dev):
    """The long causal layer at full size with the planted row at each of PLANTED: every
    output of the planted head against the oracle, to the bf16 bars (dK within 5e-2 of
    its max-norm); the margins are printed."""
    w0 = _full("long_causal")
    draws = draw_f32(w0, with_do=True)
    base = finish_inputs({n: draws[n] for n in ("k", "v", "do")}, w0)
    k, v, do = (base[n].to(dev) for n in ("k", "v", "do"))
    worst = 0.0
    for (b, h, row) in PLANTED:
        w = w0.with_(planted=(b, h, row, 30.0))
        say(f"[planted] row {row} of head ({b},{h})")
        xq = finish_inputs({"q": draws["q"]}, w)["q"]
        q = xq.to(dev)
        o, lse = fa.fwd(q, k, v, w.scale, True)
        dq, dk, dv = fa.bwd(q, k, v, o, do, lse, w.scale, True)
        torch.cuda.synchronize()
        Q = to_f64(xq[b:b + 1, h:h + 1])
        K, V, dO = (to_f64(base[n][b:b + 1, h:h + 1]) for n in ("k", "v", "do"))
        O_ref, lse_ref = attention_fwd(Q, K, V, w.scale, True)
        check_fwd("bf16", o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], O_ref, lse_ref, f"planted {row}")
        refs = attention_bwd(Q, K, V, dO, w.scale, True)
        errs = {n: check_grad("bf16", G[b:b + 1, h:h + 1], R, n, f"planted ({b},{h},{row})")
                for n, G, R in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs)}
        say(f"  dQ {errs['dQ']:.4f} dK {errs['dK']:.4f} dV {errs['dV']:.4f} (bar 0.05)")
        worst = max(worst, errs["dK"])
    say(f"[planted] worst dK relative error {worst:.4f}")


def test_fwd_bitwise_deterministic(dev):
    w = Workload("det", 2, 4, 777, 128, True, "bf16", False, seed=5)
    say("[determinism] fwd twice")
    x = make_inputs(w)
    _, _, _, o1, l1 = gpu_fwd(x, w, dev)
    _, _, _, o2, l2 = gpu_fwd(x, w, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_bwd_bitwise_deterministic(dev, d):
    """The bf16 backward accumulates without atomics: two runs agree bit for bit (the fp32
    path's dQ atomics may differ in the last bits)."""
    w = Workload("detb", 2, 3, 555, d, True, "bf16", True, seed=6)
    say(f"[determinism] bf16 bwd twice, d={d}")
    x = make_inputs(w, with_do=True)
    q, k, v, o, lse = gpu_fwd(x, w, dev)
    do = x["do"].to(dev)
    g1 = gpu_bwd(q, k, v, o, lse, do, w, dev)
    g2 = gpu_bwd(q, k, v, o, lse, do, w, dev)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_invalid_arguments_fail_loudly(dev):
    say("[errors] invalid arguments through the C ABI")
    q = torch.randn(1, 1, 64, 96, device=dev, dtype=torch.bfloat16)
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.randn(1, 1, 64, 64, device=dev, dtype=torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 64, device=dev)
    L = fa.lib()
    st = L.fa_fwd(q.data_ptr() + 2, q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(),
                  1, 1, 64, 64, 0.125, 0, fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        fa.fwd(q.half(), q.half(), q.half())


def test_autograd_saves_linear_memory(dev):
    """What the fused method keeps for backward at N=1000, d=64, fp32: Q, K, V, O
    and the lse, 1,028,000 bytes ("FlashAttention and online softmax", section 5)."""
    from saved_bytes import saved_storage_bytes

    say("[saved bytes] N=1000 d=64 fp32")
    gen = torch.Generator(device=dev).manual_seed(0)
    x = [torch.randn(1, 1, 1000, 64, device=dev, generator=gen).requires_grad_() for _ in range(3)]
    out = fa.attention(*x)
    assert saved_storage_bytes(out) == 1028000
    out.sum().backward()
    assert all(torch.isfinite(t.grad).all().item() for t in x)


@pytest.mark.timeout(300)
def test_memory_stays_linear_long_context(dev):
    """N=16384, d=128, 16 heads: the device memory high-water mark of fwd+bwd is the
    O(N) buffers, far below the 8 GiB one materialised bf16 score matrix set needs."""
    w = _full("long_context")
    say("[memory] long_context fwd+bwd")
    x = make_inputs(w)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    o, lse = fa.fwd(q, k, v, w.scale, True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, w.scale, True)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev) - base
    tensor = q.numel() * q.element_size()
    ws = fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype)
    expect = 4 * tensor + lse.numel() * 4 + ws  # o, dq, dk, dv + lse + workspace
    assert peak <= expect + (8 << 20), (peak, expect)
    assert peak < (8 << 30) // 8


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_stages_equal_fa_bwd(dev, dtype, d):
    """fa_bwd_preprocess + fa_bwd_main + fa_bwd_dq, fa_bwd's own launches one by one
    through fa_bwd_ex_launches (bf16: the dQ pass with the preprocess folded in, then the
    dK/dV pass) and, for bf16, the entry points fa_bwd_dq_pre then fa_bwd_main all
    reproduce fa_bwd bit for bit (fp32 dQ: up to its atomics' summation order)."""
    w = Workload("stages", 1, 3, 500, d, True, dtype, True, seed=7)
    say(f"[stages] bwd in separate calls vs one, {dtype} d={d}")
    x = make_inputs(w)
    q, k, v, o, lse = gpu_fwd(x, w, dev)
    do = x["do"].to(dev)
    dq1, dk1, dv1 = fa.bwd(q, k, v, o, do, lse, w.scale, True)
    for fused in (False, True):
        ws = torch.full((fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype),), 0xFF, dtype=torch.uint8,
                        device=dev)
        grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        for stage in fa.bwd_stages(q, k, v, o, do, lse, w.scale, True, ws, grads, fused=fused):
            stage()
        torch.cuda.synchronize()
        dq2, dk2, dv2 = grads
        assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2), f"fused={fused}"
        if dtype == "bf16":
            assert torch.equal(dq1, dq2), f"fused={fused}"
        else:
            check_grad("fp32", dq2, f64(dq1), "dQ", "stages")
    if dtype == "bf16":
        L, st = fa.lib(), torch.cuda.current_stream().cuda_stream
        ws = torch.full((fa.workspace_bytes(w.B, w.H, w.N, w.d, q.dtype),), 0xFF, dtype=torch.uint8, device=dev)
        dq3, dk3, dv3 = (torch.full_like(q, float("nan")) for _ in range(3))
        P = lambda t: t.data_ptr()
        wn = ws.numel()
        assert L.fa_bwd_dq_pre(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq3), P(ws), wn, w.B, w.H, w.N, w.d,
                               w.scale, 1, fa.FA_DTYPE_BF16, st) == fa.FA_OK
        assert L.fa_bwd_main(P(q), P(k), P(v), P(do), P(dk3), P(dv3), P(ws), wn, w.B, w.H, w.N, w.d,
                             w.scale, 1, fa.FA_DTYPE_BF16, st) == fa.FA_OK
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq3) and torch.equal(dk1, dk3) and torch.equal(dv1, dv3)


def test_calls_run_on_the_current_stream(dev):
    """The binding enqueues on torch's current stream.  On a side stream (default
    priority), a chain of large matrix products and then a copy into q and dO are
    queued ahead of fa.fwd / fa.bwd.  Kernels launched on any other stream would start
    before the copy lands and read zeros.  Results must equal those of the same calls on
    the default stream, bit for bit."""
    w = Workload("stream", 1, 2, 700, 128, True, "bf16", True, seed=5)
    say("[stream] fwd + bwd queued behind a copy on a side stream")
    x = make_inputs(w)
    q, k, v, o_ref, lse_ref = gpu_fwd(x, w, dev)
    do = x["do"].to(dev)
    dq_ref, dk_ref, dv_ref = fa.bwd(q, k, v, o_ref, do, lse_ref, w.scale, True)
    qs, dos = torch.zeros_like(q), torch.zeros_like(do)
    a = torch.randn(4096, 4096, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        for _ in range(8):  # keeps the side stream busy for several milliseconds
            torch.mm(a, a, out=b)
            torch.mm(b, b, out=a)
        qs.copy_(q)
        dos.copy_(do)
        o, lse = fa.fwd(qs, k, v, w.scale, True)
        dq, dk, dv = fa.bwd(qs, k, v, o, dos, lse, w.scale, True)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert torch.equal(dq, dq_ref) and torch.equal(dk, dk_ref) and torch.equal(dv, dv_ref)


@pytest.mark.timeout(600)
def test_very_long_sequence(dev):
    """One head of 131072 tokens, d = 128, causal, bf16 (eight times a long-context
    head; its score matrix would take 32 GiB in bf16): forward and backward run, every
    output is finite, and sampled rows of O and lse match the oracle row by row (one
    query against the keys it sees), including rows at tile boundaries and the last."""
    w = Workload("very_long", 1, 1, 131072, 128, True, "bf16", True, seed=11)
    say(f"[very long] N={w.N} d={w.d} causal bf16")
    x = make_inputs(w)
    q, k, v, o, lse = gpu_fwd(x, w, dev)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, x["do"].to(dev), w, dev)
    torch.cuda.synchronize()
    for G in (o, lse, dq, dk, dv):
        assert torch.isfinite(G).all().item()
    rng = np.random.default_rng(5)
    rows = sorted({0, 1, 63, 64, 255, 256, 4095, 65535, 65536, w.N - 2, w.N - 1,
                   *rng.integers(0, w.N, size=8).tolist()})
    Q, K, V = (to_f64(x[n]) for n in ("q", "k", "v"))
    for i in rows:
        O_ref, lse_ref = attention_fwd_rect(Q[:, :, i:i + 1], K[:, :, :i + 1], V[:, :, :i + 1],
                                            w.scale, True)
        check_fwd("bf16", o[:, :, i:i + 1], lse[:, :, i:i + 1], O_ref, lse_ref, f"row {i}")
    say(f"  {len(rows)} sampled rows match")


def test_binding_rejects_bad_output_buffers(dev):
    """Caller-supplied outputs of the wrong shape, dtype, device or layout raise
    ValueError in the binding, before anything is enqueued (the C ABI cannot see
    buffer sizes)."""
    say("[errors] output buffers checked by the binding")
    B, H, N, d = 1, 2, 64, 64
    q = torch.randn(B, H, N, d, device=dev, dtype=torch.bfloat16)
    o, lse = fa.fwd(q, q, q)
    bad_outs = [torch.empty(B, H, N, d // 2, device=dev, dtype=torch.bfloat16),  # short
                torch.empty(B, H, N, d, device=dev, dtype=torch.float32),       # dtype
                torch.empty(B, H, N, d, dtype=torch.bfloat16),                  # host memory
                torch.empty(B, H, d, N, device=dev, dtype=torch.bfloat16).transpose(2, 3)]
    bad_lse = [torch.empty(B, H, device=dev), torch.empty(B, H, N, device=dev, dtype=torch.bfloat16),
               torch.empty(B, H, N)]
    for t in bad_outs:
        with pytest.raises(ValueError):
            fa.fwd(q, q, q, out=t)
        with pytest.raises(ValueError):
            fa.bwd(q, q, q, o, q, lse, grads=(torch.empty_like(q), t, torch.empty_like(q)))
    for t in bad_lse:
        with pytest.raises(ValueError):
            fa.fwd(q, q, q, lse=t)
        with pytest.raises(ValueError):
            fa.bwd(q, q, q, o, q, t)
    with pytest.raises(ValueError):  # workspace too short
        fa.bwd(q, q, q, o, q, lse, workspace=torch.empty(16, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):  # fwd_ex output
        fa.fwd_ex(q, q, q, causal=True, window=4, out=bad_outs[0])
    qd = torch.randn(B, H, 1, d, device=dev, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # split-KV partials of the wrong shape
        fa.fwd_partial(qd, q, q, 4, o_part=torch.empty(4, B, H, 1, d // 2, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_partial(qd, q, q, 4, lse_part=torch.empty(4, B, H, device=dev))
    op, lp = fa.fwd_partial(qd, q, q, 4)
    with pytest.raises(ValueError):  # merge output of the wrong dtype / shape
        fa.merge(op, lp, torch.bfloat16, out=torch.empty(B, H, 1, d, device=dev))
    with pytest.raises(ValueError):
        fa.merge(op, lp, torch.float32, lse=torch.empty(B, H, 2, device=dev))
    torch.cuda.synchronize()
