"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only draws random numbers, applies
the planted-row structure and rounds to the storage dtype.  Both the HIP path
(tests, benchmark) and the CPU oracle receive the arrays it returns, so the oracle
sees exactly the values the GPU sees.

Recipe (shared by every workload):
  rng = numpy.random.default_rng(seed); draw Q, K, V, dO in that order, each
  ``rng.standard_normal((B, H, N, d), dtype=float32)`` in C order; optionally scale
  one query row by a constant (the planted row) before rounding; round to bf16 with
  round-to-nearest-even (torch CPU ``.to(torch.bfloat16)``) unless the workload is
  fp32.  The softmax scale is 1/sqrt(d).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "draw_f32", "finish_inputs", "to_f64",
           "DecodeWorkload", "DECODE_WORKLOADS", "make_decode_inputs",
           "WINDOW_WORKLOADS", "VarlenWorkload", "VARLEN_WORKLOADS", "varlen_lengths",
           "make_varlen_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str  # "bf16" or "fp32"
    backward: bool
    planted: tuple | None = None  # (b, h, row, factor) applied to Q before rounding
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads: shapes, masks and dtypes as the attention layers they stand in for.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 256, 64, False, "fp32", True),
    "gpt2m_fwd": Workload("gpt2m_fwd", 8, 16, 1024, 64, False, "bf16", False),
    "long_causal": Workload("long_causal", 4, 32, 4096, 128, True, "bf16", True,
                            planted=(0, 0, 2049, 30.0)),
    "train_step": Workload("train_step", 4, 16, 2048, 64, True, "bf16", True),
    "long_context": Workload("long_context", 1, 16, 16384, 128, True, "bf16", True),
}


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t.to(torch.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_f32(w: Workload, with_do: bool | None = None) -> dict:
    """The workload's float32 draws before any planting or rounding: dict q, k, v[, do]
    of numpy arrays (the first steps of the recipe)."""
    if with_do is None:
        with_do = w.backward
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    return {name: rng.standard_normal(shape, dtype=np.float32) for name in names}


def finish_inputs(draws: dict, w: Workload) -> dict:
    """The recipe's last steps on draws from draw_f32: scale the planted query row of
    ``w.planted`` (on a copy of q), then round every tensor to ``w.dtype``."""
    out = {}
    for name, x in draws.items():
        if name == "q" and w.planted is not None:
            b, h, row, factor = w.planted
            if b < w.B and h < w.H and row < w.N:
                x = x.copy()
                x[b, h, row, :] *= np.float32(factor)
        out[name] = _round(x, w.dtype)
    return out


def make_inputs(w: Workload, with_do: bool | None = None) -> dict:
    """Draw the workload's tensors. Returns dict q, k, v[, do] of CPU torch tensors."""
    return finish_inputs(draw_f32(w, with_do), w)


@dataclass(frozen=True)
class DecodeWorkload:
    """Nq new query rows per (b, h) against a cache of Nk key/value rows."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str
    splits: int
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# Decoding with a long cache at the shape of the pages' split-KV example (batch 4,
# 16 heads, one new token), head dim 128, cache of 16384 tokens; split into 16
# chunks (1024 workgroups, four per compute unit).
DECODE_WORKLOADS = {
    "decode_long": DecodeWorkload("decode_long", 4, 16, 1, 16384, 128, True, "bf16", 16),
}


def make_decode_inputs(w: DecodeWorkload) -> dict:
    """Same recipe as make_inputs: q [B,H,Nq,d], then k, v [B,H,Nk,d], drawn in that order."""
    rng = np.random.default_rng(w.seed)
    out = {}
    for name, n in (("q", w.Nq), ("k", w.Nk), ("v", w.Nk)):
        out[name] = _round(rng.standard_normal((w.B, w.H, n, w.d), dtype=np.float32), w.dtype)
    return out


# Long-context training with a sliding window: the long-context shape (1 x 16 heads,
# N = 16384, d = 128, causal) with a band of 4096 keys.
WINDOW_WORKLOADS = {
    "window_long": (Workload("window_long", 1, 16, 16384, 128, True, "bf16", True), 4096),
}


@dataclass(frozen=True)
class VarlenWorkload:
    """A batch of `n_seqs` sequences packed head-major [H, T, d], lengths drawn
    log-uniform in [min_len, max_len] (rounded)."""
    name: str
    n_seqs: int
    min_len: int
    max_len: int
    H: int
    d: int
    causal: bool
    dtype: str
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


VARLEN_WORKLOADS = {
    "varlen_mix": VarlenWorkload("varlen_mix", 16, 256, 4096, 16, 128, True, "bf16"),
}


def varlen_lengths(w: VarlenWorkload) -> np.ndarray:
    """Sequence lengths: rng = default_rng(seed + 1); exp(uniform(log min, log max)),
    rounded to integers."""
    rng = np.random.default_rng(w.seed + 1)
    x = rng.uniform(math.log(w.min_len), math.log(w.max_len), size=w.n_seqs)
    return np.rint(np.exp(x)).astype(np.int64)


def make_varlen_inputs(w: VarlenWorkload, lengths=None, with_do: bool = True) -> dict:
    """q, k, v[, do] packed [H, T, d] and cu_seqlens (int32, [B+1]); the draws follow
    make_inputs' recipe with shape (H, T, d)."""
    lens = varlen_lengths(w) if lengths is None else np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(w.seed)
    out = {"cu": torch.from_numpy(cu), "max_len": int(lens.max()) if len(lens) else 0}
    for name in ["q", "k", "v"] + (["do"] if with_do else []):
        out[name] = _round(rng.standard_normal((w.H, int(cu[-1]), w.d), dtype=np.float32), w.dtype)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 CPU tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()
