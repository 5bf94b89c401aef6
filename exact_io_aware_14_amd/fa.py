"""ctypes binding of libfa.so (exact tiled attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/fa.h``.  PyTorch supplies device memory and
the current stream.  There is no fallback: if the library is missing or a call is
rejected, these functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["lib", "fwd", "bwd", "bwd_stages", "workspace_bytes", "attention", "FaError",
           "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_LAUNCH",
           "FA_DTYPE_BF16", "FA_DTYPE_FP32", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH = 0, 1, 2, 3
FA_DTYPE_BF16, FA_DTYPE_FP32 = 0, 1

_DTYPES = {torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_FP32}


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().fa_status_string(status).decode()} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_io_aware_14_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m exact_io_aware_14_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        L.fa_fwd.restype = i
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
        L.fa_bwd.restype = i
        L.fa_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, i, vp]
        L.fa_bwd_preprocess.restype = i
        L.fa_bwd_main.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
        L.fa_bwd_main.restype = i
        L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
        L.fa_bwd_dq.restype = i
        L.fa_fwd_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i]
        L.fa_fwd_check.restype = i
        L.fa_bwd_check.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i]
        L.fa_bwd_check.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_abi_version.argtypes = []
        L.fa_abi_version.restype = i
        _lib = L
    return _lib


def _dims(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _check_same(*ts: torch.Tensor):
    t0 = ts[0]
    for t in ts:
        if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError("all [B, H, N, d] tensors must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    if t0.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    if t0.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t0.dtype} (bf16 or float32)")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def workspace_bytes(B: int, H: int, N: int, d: int, dtype: torch.dtype) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d, _DTYPES[dtype]))


def fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None):
    """O, lse = attention forward.  q, k, v: contiguous [B, H, N, d] bf16/fp32 on the GPU."""
    _check_same(q, k, v)
    B, H, N, d = _dims(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                      B, H, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype], _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return o, l


def bwd(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False,
        workspace=None, grads=None):
    """dQ, dK, dV of sum(do * o).  ``lse`` is the fp32 output of :func:`fwd`."""
    _check_same(q, k, v, o, do)
    B, H, N, d = _dims(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    nbytes = workspace_bytes(B, H, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    st = lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                      B, H, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype],
                      _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def bwd_stages(q, k, v, o, do, lse, scale, causal, workspace, grads):
    """The three stages of :func:`bwd` as separate calls (same result), returning a
    list of three callables so a caller can time or interleave them."""
    _check_same(q, k, v, o, do)
    B, H, N, d = _dims(q)
    dq, dk, dv = grads
    L, dt, st = lib(), _DTYPES[q.dtype], _stream(q.device)
    wp, wn = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    sc, ca = float(scale), int(bool(causal))

    def pre():
        r = L.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), wp, wn, B, H, N, d, dt, st)
        if r != FA_OK:
            raise FaError(r, "fa_bwd_preprocess")

    def main():
        r = L.fa_bwd_main(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                          dk.data_ptr(), dv.data_ptr(), wp, wn, B, H, N, d, sc, ca, dt, st)
        if r != FA_OK:
            raise FaError(r, "fa_bwd_main")

    def dqs():
        r = L.fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), dq.data_ptr(),
                        wp, wn, B, H, N, d, sc, ca, dt, st)
        if r != FA_OK:
            raise FaError(r, "fa_bwd_dq")

    return [pre, main, dqs]


class _Attention(torch.autograd.Function):
    """Autograd wrapper: saves q, k, v, o and the fp32 lse -- O(N) per head."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        o, lse = fwd(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, do.contiguous(), lse, ctx.scale, ctx.causal)
        return dq, dk, dv, None, None


def attention(q, k, v, scale: float | None = None, causal: bool = False):
    """Differentiable exact attention on [B, H, N, d] tensors."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _Attention.apply(q, k, v, scale, causal)
