"""GPU parity of split-KV decoding (fa_fwd_partial, fa_merge, fa_fwd_splitkv)
against the CPU fp64 oracle (oracle/splitkv.py).

Bars: partial outputs are float32 sums of exact products, so o_part and lse_part
agree with the oracle to 1e-5 (relative to the row's max |o|, and absolute on lse)
for both input types; the merged O takes the forward's bar for its dtype (fp32:
1e-5 relative; bf16: 2e-2 absolute) and lse 1e-5 (fp32) / 1e-3 (bf16).
"""
import numpy as np
import pytest
import torch

from exact_io_aware_14_amd import fa
from exact_io_aware_14_amd.inputs import DECODE_WORKLOADS, DecodeWorkload, make_decode_inputs, to_f64
from oracle import attention_fwd_rect, merge_partials, splitkv_partials
from parity import check_fwd

pytestmark = pytest.mark.gpu
TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.lib()
    return torch.device("cuda:0")


def check_partials(op, lp, op_ref, lp_ref, label):
    op, lp = op.cpu().double().numpy(), lp.cpu().double().numpy()
    assert op.shape == op_ref.shape and lp.shape == lp_ref.shape
    empty = lp_ref == -np.inf
    assert np.array_equal(lp == -np.inf, empty), f"{label}: empty partials differ"
    assert np.all(op[empty] == 0.0), f"{label}: empty partial o not zero"
    fin = ~empty
    if fin.any():
        el = np.abs(lp[fin] - lp_ref[fin]).max()
        assert el <= 1e-5 * max(1.0, np.abs(lp_ref[fin]).max()), f"{label}: lse_part err {el:.3e}"
        eo = np.abs(op - op_ref).max() / max(np.abs(op_ref).max(), 1e-30)
        assert eo <= 1e-5, f"{label}: o_part rel err {eo:.3e}"


CASES = [  # B, H, Nq, Nk, splits
    (1, 1, 1, 1, 1), (2, 3, 1, 300, 4), (1, 2, 3, 1000, 7), (2, 2, 8, 513, 16),
    (1, 1, 1, 37, 64), (1, 2, 5, 5, 2), (1, 1, 2, 2048, 1), (2, 1, 4, 777, 256)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dq%dk%ds%d" % c)
def test_small_splitkv(dev, dtype, d, causal, case):
    B, H, Nq, Nk, S = case
    w = DecodeWorkload("small", B, H, Nq, Nk, d, causal, dtype, S, seed=Nk + 7 * Nq + d)
    say(f"[splitkv] {dtype} B={B} H={H} Nq={Nq} Nk={Nk} d={d} S={S} causal={causal}")
    x = make_decode_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    Q, K, V = (to_f64(x[n]) for n in ("q", "k", "v"))
    op = torch.full((S, B, H, Nq, d), float("nan"), device=dev)
    lp = torch.full((S, B, H, Nq), float("nan"), device=dev)
    fa.fwd_partial(q, k, v, S, w.scale, causal, o_part=op, lse_part=lp)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device=dev)
    fa.fwd_splitkv(q, k, v, S, w.scale, causal, out=o, lse=lse)
    torch.cuda.synchronize()
    op_ref, lp_ref = splitkv_partials(Q, K, V, w.scale, causal, S)
    check_partials(op, lp, op_ref, lp_ref, "partials")
    O_ref, lse_ref = attention_fwd_rect(Q, K, V, w.scale, causal)
    check_fwd(dtype, o.cpu(), lse.cpu(), O_ref, lse_ref, "merged")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_merge_alone(dev, dtype):
    """fa_merge on random partials with empty chunks and wholly empty rows."""
    rng = np.random.default_rng(11)
    S, rows, d = 9, 50, 96
    op = rng.standard_normal((S, rows, d))
    lp = 3.0 * rng.standard_normal((S, rows))
    lp[rng.random((S, rows)) < 0.3] = -np.inf
    lp[:, 7] = -np.inf  # a row with no key at all
    op[lp == -np.inf] = 0.0
    o, l = fa.merge(torch.tensor(op, dtype=torch.float32, device=dev),
                    torch.tensor(lp, dtype=torch.float32, device=dev), TORCH_DT[dtype])
    torch.cuda.synchronize()
    opf, lpf = op.astype(np.float32).astype(np.float64), lp.astype(np.float32).astype(np.float64)
    O_ref, lse_ref = merge_partials(opf, lpf)
    assert np.all(l.cpu().numpy()[7] == -np.inf) and np.all(o.cpu().float().numpy()[7] == 0.0)
    keep = np.arange(rows) != 7
    check_fwd(dtype, o.cpu()[keep], l.cpu()[keep], O_ref[keep], lse_ref[keep], "merge")


@pytest.mark.parametrize("splits", [1, 8, 32])
def test_decode_long_full_size(dev, splits):
    """The decoding workload at its real size (the pages' batch-4, 16-head example
    with a 16384-token cache), every row against the oracle."""
    w = DECODE_WORKLOADS["decode_long"]
    say(f"[decode_long] splits={splits}")
    x = make_decode_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd_splitkv(q, k, v, splits, w.scale, w.causal)
    torch.cuda.synchronize()
    O_ref, lse_ref = attention_fwd_rect(*(to_f64(x[n]) for n in ("q", "k", "v")), w.scale, w.causal)
    check_fwd(w.dtype, o.cpu(), lse.cpu(), O_ref, lse_ref, f"decode_long S={splits}")


def test_splitkv_invalid_args(dev):
    q = torch.zeros((1, 1, 9, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, 20, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError) as e:
        fa.fwd_splitkv(q, k, k, 4)  # Nq > 8
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q1 = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device=dev)
    k3 = torch.zeros((1, 1, 3, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError) as e:
        fa.fwd_splitkv(q1, k3, k3, 2)  # Nk < Nq
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    with pytest.raises(fa.FaError) as e:
        fa.fwd_partial(q1, k, k, 0)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    with pytest.raises(fa.FaError) as e:
        fa.fwd_partial(q1, k, k, 257)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):  # the binding checks the workspace's size first
        fa.fwd_splitkv(q1, k, k, 4, workspace=small)
    o = torch.empty_like(q1)
    lse = torch.empty((1, 1, 4), dtype=torch.float32, device=dev)
    st = fa.lib().fa_fwd_splitkv(q1.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 1, 1, 4, 20, 64, 0.125, 1, 4, small.data_ptr(), 16, fa.FA_DTYPE_BF16,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_INVALID_ARG  # and so does the C ABI, before any launch
