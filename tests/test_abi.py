"""The C-ABI library loads, exports every symbol include/fa.h declares, and its
host-side argument checks return the documented codes (no device is touched)."""
import ctypes
import os
import re

import pytest

from exact_io_aware_14_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH),
                                reason="libfa.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(fa_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string",
                          "fa_fwd_check", "fa_bwd_check", "fa_abi_version", "fa_bwd_preprocess",
                          "fa_bwd_main", "fa_bwd_dq", "fa_bwd_noalloc"}
    L = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = fa.lib()
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_LAUNCH,
                 fa.FA_ERR_TOO_LARGE):
        assert L.fa_status_string(code) and L.fa_status_string(code) != b"unknown status"
    assert L.fa_status_string(99) == b"unknown status"
    assert L.fa_abi_version() >> 16 == 1


P = 0x100000  # a 16-byte-aligned fake address: the checks never dereference it


def fwd_check(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=100, d=64, scale=0.125, causal=0, dtype=0)
    a.update(kw)
    return fa.lib().fa_fwd_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                 a["d"], a["scale"], a["causal"], a["dtype"])


def bwd_check(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, wsb=1 << 30, B=1, H=2,
             N=100, d=64, scale=0.125, causal=1, dtype=0)
    a.update(kw)
    L = fa.lib()
    return L.fa_bwd_check(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                          a["dv"], a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                          a["causal"], a["dtype"])


def test_fwd_check_codes():
    assert fwd_check() == fa.FA_OK
    assert fwd_check(d=128, dtype=1, causal=1) == fa.FA_OK
    for bad in (dict(q=None), dict(lse=None), dict(B=0), dict(H=-1), dict(N=0),
                dict(q=P + 8), dict(o=P + 2), dict(lse=P + 2), dict(scale=0.0), dict(scale=-1.0),
                dict(scale=float("inf")), dict(scale=float("nan")), dict(causal=2),
                dict(B=1 << 16, H=1 << 10, N=1 << 10)):
        assert fwd_check(**bad) == fa.FA_ERR_INVALID_ARG, bad
    for bad in (dict(d=96), dict(d=256), dict(d=32), dict(dtype=2), dict(dtype=-1)):
        assert fwd_check(**bad) == fa.FA_ERR_UNSUPPORTED, bad


def test_bwd_check_codes_and_workspace():
    L = fa.lib()
    ws = L.fa_bwd_workspace_bytes(1, 2, 100, 64, 0)
    padded = 2 * 128  # N = 100 padded to a multiple of 32 per head
    rnd = lambda x: (x + 255) // 256 * 256
    plan = rnd(4 * (16 + 2 * 1))  # block plan: header + one id per 128 keys of each head
    assert ws == 2 * rnd(padded * 4) + plan  # bf16: D and lse vectors, plan
    assert L.fa_bwd_workspace_bytes(1, 2, 100, 64, 1) == 2 * rnd(padded * 4) + rnd(padded * 64 * 4) + plan
    assert L.fa_bwd_workspace_bytes(1, 2, 100, 96, 0) == 0
    assert bwd_check(wsb=ws) == fa.FA_OK
    assert bwd_check(wsb=ws - 1) == fa.FA_ERR_INVALID_ARG
    for bad in (dict(do=None), dict(ws=None), dict(dk=P + 4), dict(ws=P + 8), dict(causal=-1)):
        assert bwd_check(**bad) == fa.FA_ERR_INVALID_ARG, bad
    assert bwd_check(d=80) == fa.FA_ERR_UNSUPPORTED


def test_entry_points_reject_before_touching_the_device():
    """fa_fwd / fa_bwd run the same checks first and launch nothing on failure."""
    L = fa.lib()
    assert L.fa_fwd(P, P, P, P, P, 1, 1, 10, 96, 0.1, 0, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_fwd(None, P, P, P, P, 1, 1, 10, 64, 0.1, 0, 0, None) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd(P, P, P, P, P, P, P, P, P, P, 0, 1, 1, 10, 64, 0.1, 0, 0, None) == fa.FA_ERR_INVALID_ARG


def test_noalloc_size_limit_is_checked_on_the_host():
    """fa_bwd_noalloc refuses a call whose workspace would exceed its fixed scratch
    (FA_NOALLOC_SCRATCH_BYTES, 32 MiB) before touching any device, and runs fa_bwd's
    argument checks first."""
    L = fa.lib()
    limit = 32 << 20
    assert "FA_NOALLOC_SCRATCH_BYTES (32u << 20)" in open(HEADER).read()
    B, H, N, d = 64, 64, 1056, 64  # bf16: 2 x 4.3M padded rows of 4 bytes
    assert L.fa_bwd_workspace_bytes(B, H, N, d, 0) > limit
    assert L.fa_bwd_workspace_bytes(64, 64, 1024, 64, 0) > limit  # 32 MiB of vectors + plan
    assert L.fa_bwd_workspace_bytes(64, 63, 1024, 64, 0) <= limit
    args = lambda B, H, N, d, dt: (P, P, P, P, P, P, P, P, P, B, H, N, d, 0.125, 1, dt, None)
    assert L.fa_bwd_noalloc(*args(B, H, N, d, 0)) == fa.FA_ERR_TOO_LARGE
    # fp32 adds a [B, H, Npad, d] accumulator: 4 x 32 x 1024 rows x 520 bytes > 32 MiB
    assert L.fa_bwd_noalloc(*args(4, 32, 1024, 128, 1)) == fa.FA_ERR_TOO_LARGE
    assert L.fa_bwd_noalloc(None, *args(1, 1, 64, 64, 0)[1:]) == fa.FA_ERR_INVALID_ARG
    assert L.fa_bwd_noalloc(*args(1, 1, 64, 96, 0)) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_status_string(fa.FA_ERR_TOO_LARGE) != b"unknown status"


def test_bwd_ex_launches_mask_checked_on_the_host():
    L = fa.lib()
    for mask in (0, 8, -1):
        assert L.fa_bwd_ex_launches(P, P, P, P, P, P, P, P, P, P, 1 << 30, None, 1, 2, 100, 0, 64, 0.125,
                                    1, 0, 0, mask, None) == fa.FA_ERR_INVALID_ARG
