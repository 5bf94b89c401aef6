"""fa_bwd_noalloc (the backward without a workspace argument, for callers that cannot
allocate) against fa_bwd, through the C ABI, on two calls in a row: the second one
smaller (fewer heads, shorter, other head dim), so it runs on what the first call
left in the library's scratch."""
import pytest
import torch

from exact_io_aware_14_amd import fa
from exact_io_aware_14_amd.inputs import Workload, make_inputs
from parity import f64, maxabs

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.lib()
    return torch.device("cuda:0")


def noalloc(q, k, v, o, do, lse, grads, scale, causal):
    B, H, N, d = (int(x) for x in q.shape)
    return fa.lib().fa_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), B, H, N, d, float(scale),
        int(causal), fa._DTYPES[q.dtype], torch.cuda.current_stream(q.device).cuda_stream)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_equals_fa_bwd_on_two_calls(dev, dtype):
    # (B, H, N, d, causal): the second call is smaller than the first
    for i, (B, H, N, d, causal) in enumerate([(2, 3, 300, 128, True), (1, 2, 90, 64, False)]):
        print(f"[noalloc] {dtype} call {i}: B={B} H={H} N={N} d={d} causal={causal}", flush=True)
        w = Workload(f"noalloc{i}", B, H, N, d, causal, dtype, True, seed=7 + i)
        x = make_inputs(w)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = fa.fwd(q, k, v, w.scale, causal)
        ref = fa.bwd(q, k, v, o, do, lse, w.scale, causal)
        got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        assert noalloc(q, k, v, o, do, lse, got, w.scale, causal) == fa.FA_OK
        torch.cuda.synchronize()
        for name, G, R in zip(("dQ", "dK", "dV"), got, ref):
            if dtype == "bf16":  # same kernels, deterministic: bit for bit
                assert torch.equal(G, R), f"call {i} {name} differs from fa_bwd"
            else:  # fp32 dQ sums with atomics: equal up to the fp32 bar
                e, r = maxabs(f64(G) - f64(R)), maxabs(f64(R))
                assert e <= 1e-5 * r, f"call {i} {name}: {e:.3e} vs {r:.3e}"


def test_noalloc_rejects_what_does_not_fit(dev):
    """A call whose workspace exceeds the fixed scratch is refused before any launch."""
    B, H, N, d = 64, 64, 1056, 64  # bf16: 2 x 4.3M rows of 4 bytes > 32 MiB
    assert fa.lib().fa_bwd_workspace_bytes(B, H, N, d, 0) > (32 << 20)
    P = 0x100000
    st = fa.lib().fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, B, H, N, d, 0.125, 1, 0, None)
    assert st == fa.FA_ERR_TOO_LARGE
