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
           "fwd_splitkv", "fwd_partial", "merge", "splitkv_workspace_bytes", "fwd_ex", "bwd_ex",
           "bwd_noalloc", "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_LAUNCH",
           "FA_ERR_TOO_LARGE",
           "FA_DTYPE_BF16", "FA_DTYPE_FP32", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
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
        L.fa_bwd_dq_pre.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
        L.fa_bwd_dq_pre.restype = i
        L.fa_fwd_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i]
        L.fa_fwd_check.restype = i
        L.fa_bwd_check.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i]
        L.fa_bwd_check.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
        L.fa_fwd_ex.restype = i
        L.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, f, i, i,
                                i, vp]
        L.fa_bwd_ex.restype = i
        L.fa_bwd_ex_launches.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, f,
                                         i, i, i, i, vp]
        L.fa_bwd_ex_launches.restype = i
        L.fa_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_splitkv_workspace_bytes.restype = sz
        L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, i, vp]
        L.fa_fwd_splitkv.restype = i
        L.fa_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
        L.fa_fwd_partial.restype = i
        L.fa_merge.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        L.fa_merge.restype = i
        L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        L.fa_bwd_noalloc.restype = i
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


def _out(t, shape, dtype, device, name):
    """A caller-supplied output buffer, checked before the library sees it: the C ABI
    cannot see buffer sizes, so a short or mistyped buffer would be written past its
    end on the device.  Returns ``t``."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(ws, device, need: int):
    """A caller-supplied workspace: contiguous device memory of at least ``need`` bytes."""
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws


def _grads(grads, like):
    if grads is None:
        return tuple(torch.empty_like(like) for _ in range(3))
    if len(grads) != 3:
        raise ValueError("grads must be (dq, dk, dv)")
    return tuple(_out(g, like.shape, like.dtype, like.device, n) for g, n in zip(grads, ("dq", "dk", "dv")))


def workspace_bytes(B: int, H: int, N: int, d: int, dtype: torch.dtype) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d, _DTYPES[dtype]))


def fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None):
    """O, lse = attention forward.  q, k, v: contiguous [B, H, N, d] bf16/fp32 on the GPU."""
    _check_same(q, k, v)
    B, H, N, d = _dims(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else _out(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
         else _out(lse, (B, H, N), torch.float32, q.device, "lse"))
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
    _out(lse, (B, H, N), torch.float32, q.device, "lse")
    nbytes = workspace_bytes(B, H, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _workspace(workspace, q.device, nbytes)
    dq, dk, dv = _grads(grads, q)
    st = lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                      B, H, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype],
                      _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False,
                grads=None):
    """:func:`bwd` through fa_bwd_noalloc: no workspace, the library's fixed scratch
    instead (calls on one GPU must not overlap; see include/fa.h)."""
    _check_same(q, k, v, o, do)
    B, H, N, d = _dims(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _out(lse, (B, H, N), torch.float32, q.device, "lse")
    dq, dk, dv = _grads(grads, q)
    st = lib().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                              B, H, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype],
                              _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def bwd_stages(q, k, v, o, do, lse, scale, causal, workspace, grads, fused: bool = False):
    """The backward as separate calls (same result as :func:`bwd`), returned as a list of
    callables so a caller can time or interleave them.  ``fused=False``: the three stages
    fa_bwd_preprocess, fa_bwd_main, fa_bwd_dq.  ``fused=True``: the launches fa_bwd itself
    makes, one call each through fa_bwd_ex_launches (bf16: the dQ pass with the
    preprocess folded in, then the dK/dV pass; fp32: the three stages)."""
    _check_same(q, k, v, o, do)
    B, H, N, d = _dims(q)
    _out(lse, (B, H, N), torch.float32, q.device, "lse")
    _workspace(workspace, q.device, workspace_bytes(B, H, N, d, q.dtype))
    dq, dk, dv = _grads(grads, q)
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

    def launch(mask):
        def run():
            r = L.fa_bwd_ex_launches(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), wp, wn,
                                     None, B, H, N, 0, d, sc, ca, 0, dt, mask, st)
            if r != FA_OK:
                raise FaError(r, "fa_bwd_ex_launches")
        return run

    if fused and q.dtype == torch.bfloat16:
        return [launch(1), launch(2)]
    return [pre, main, dqs]


def _ex_dims(q, cu_seqlens, max_seqlen, validate=True):
    """(B, H, N, total, d, lse shape, cu pointer) of a dense or packed call."""
    if cu_seqlens is None:
        B, H, N, d = _dims(q)
        return B, H, N, 0, d, (B, H, N), 0
    if q.dim() != 3:
        raise ValueError("variable-length tensors are packed [H, total, d]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 [B+1] tensor on q's device")
    if max_seqlen is None:
        raise ValueError("max_seqlen is required with cu_seqlens")
    H, T, d = (int(x) for x in q.shape)
    if validate:
        # The library reads the table on the device and cannot reject it; checked here
        # on a host copy (one device-to-host transfer), so that a table outside the
        # rules of fa_fwd_ex fails loudly instead of giving wrong rows.
        cu = cu_seqlens.cpu().tolist()
        if len(cu) < 2 or cu[0] != 0 or cu[-1] != T:
            raise ValueError(f"cu_seqlens must run from 0 to total = {T}")
        lens = [b - a for a, b in zip(cu, cu[1:])]
        if min(lens) < 0:
            raise ValueError("cu_seqlens must be non-decreasing")
        if max(lens) > int(max_seqlen):
            raise ValueError(f"a sequence of {max(lens)} tokens exceeds max_seqlen = {max_seqlen}")
    return int(cu_seqlens.numel()) - 1, H, int(max_seqlen), T, d, (H, T), cu_seqlens.data_ptr()


def fwd_ex(q, k, v, scale: float | None = None, causal: bool = False, window: int = 0,
           cu_seqlens=None, max_seqlen: int | None = None, out=None, lse=None,
           validate: bool = True):
    """Forward with a sliding window and/or variable-length packed sequences
    ([H, total, d] with int32 cu_seqlens [B+1]); see fa_fwd_ex in include/fa.h.
    ``validate`` checks cu_seqlens on a host copy first (0 = cu[0] <= ... <= cu[B] =
    total, every length <= max_seqlen); a caller that guarantees that may pass False
    to skip the device-to-host transfer."""
    _check_same(q, k, v)
    B, H, N, T, d, lshape, cu = _ex_dims(q, cu_seqlens, max_seqlen, validate)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else _out(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty(lshape, dtype=torch.float32, device=q.device) if lse is None
         else _out(lse, lshape, torch.float32, q.device, "lse"))
    st = lib().fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), cu,
                         B, H, N, T, d, float(scale), int(bool(causal)), int(window),
                         _DTYPES[q.dtype], _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_ex")
    return o, l


def bwd_ex(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False, window: int = 0,
           cu_seqlens=None, max_seqlen: int | None = None, workspace=None, grads=None,
           validate: bool = True, launches: int = 7):
    """Backward of :func:`fwd_ex` (same layout and arguments).  ``launches`` selects
    which of the backward's kernel launches to enqueue (a bit mask in their order; see
    fa_bwd_ex_launches in include/fa.h); the default runs all of them."""
    _check_same(q, k, v, o, do)
    B, H, N, T, d, lshape, cu = _ex_dims(q, cu_seqlens, max_seqlen, validate)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _out(lse, lshape, torch.float32, q.device, "lse")
    nbytes = workspace_bytes(B, H, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, q.device, nbytes)
    dq, dk, dv = _grads(grads, q)
    st = lib().fa_bwd_ex_launches(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), cu,
                                  B, H, N, T, d, float(scale), int(bool(causal)), int(window),
                                  _DTYPES[q.dtype], int(launches), _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_ex")
    return dq, dk, dv


def _check_decode(q, k, v):
    _check_same(k, v)
    if q.dim() != 4 or q.dtype != k.dtype or q.device != k.device or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, H, Nq, d] tensor of k's dtype and device")
    B, H, Nq, d = _dims(q)
    Bk, Hk, Nk, dk = _dims(k)
    if (Bk, Hk, dk) != (B, H, d):
        raise ValueError("q [B, H, Nq, d] and k, v [B, H, Nk, d] disagree on B, H or d")
    return B, H, Nq, Nk, d


def splitkv_workspace_bytes(B: int, H: int, Nq: int, d: int, num_splits: int) -> int:
    return int(lib().fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits))


def fwd_splitkv(q, k, v, num_splits: int, scale: float | None = None, causal: bool = False,
                out=None, lse=None, workspace=None):
    """Split-KV decoding: O [B,H,Nq,d], lse [B,H,Nq] of q [B,H,Nq,d] over the cache
    k, v [B,H,Nk,d] cut into ``num_splits`` chunks (partials, then their merge)."""
    B, H, Nq, Nk, d = _check_decode(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else _out(out, q.shape, q.dtype, q.device, "out")
    l = (torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None
         else _out(lse, (B, H, Nq), torch.float32, q.device, "lse"))
    n = splitkv_workspace_bytes(B, H, Nq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, q.device, n)
    st = lib().fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                              B, H, Nq, Nk, d, float(scale), int(bool(causal)), int(num_splits),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _DTYPES[q.dtype], _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv")
    return o, l


def fwd_partial(q, k, v, num_splits: int, scale: float | None = None, causal: bool = False,
                o_part=None, lse_part=None):
    """First pass of :func:`fwd_splitkv`: float32 o_part [S,B,H,Nq,d], lse_part [S,B,H,Nq]."""
    B, H, Nq, Nk, d = _check_decode(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = int(num_splits)
    op = (torch.empty((S, B, H, Nq, d), dtype=torch.float32, device=q.device) if o_part is None
          else _out(o_part, (S, B, H, Nq, d), torch.float32, q.device, "o_part"))
    lp = (torch.empty((S, B, H, Nq), dtype=torch.float32, device=q.device) if lse_part is None
          else _out(lse_part, (S, B, H, Nq), torch.float32, q.device, "lse_part"))
    st = lib().fa_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), op.data_ptr(), lp.data_ptr(),
                              B, H, Nq, Nk, d, float(scale), int(bool(causal)), S,
                              _DTYPES[q.dtype], _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_partial")
    return op, lp


def merge(o_part, lse_part, dtype: torch.dtype = torch.float32, out=None, lse=None):
    """Second pass: merge float32 partials o_part [S, ..., d], lse_part [S, ...] into
    o [..., d] of ``dtype`` and lse [...] float32."""
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise ValueError("partials are float32")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("partials must be contiguous")
    if tuple(o_part.shape[:-1]) != tuple(lse_part.shape):
        raise ValueError("o_part [S, ..., d] and lse_part [S, ...] disagree")
    S, d = int(o_part.shape[0]), int(o_part.shape[-1])
    rows = int(lse_part.numel() // max(S, 1))
    if o_part.device.type != "cuda" or lse_part.device != o_part.device:
        raise ValueError("partials must live on one GPU")
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype} (bf16 or float32)")
    oshape, lshape = tuple(o_part.shape[1:]), tuple(lse_part.shape[1:])
    o = (torch.empty(oshape, dtype=dtype, device=o_part.device) if out is None
         else _out(out, oshape, dtype, o_part.device, "out"))
    l = (torch.empty(lshape, dtype=torch.float32, device=o_part.device) if lse is None
         else _out(lse, lshape, torch.float32, o_part.device, "lse"))
    st = lib().fa_merge(o_part.data_ptr(), lse_part.data_ptr(), o.data_ptr(), l.data_ptr(),
                        S, rows, d, _DTYPES[dtype], _stream(o_part.device))
    if st != FA_OK:
        raise FaError(st, "fa_merge")
    return o, l


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
