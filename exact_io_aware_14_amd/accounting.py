"""FLOP and byte accounting for the attention hot path (host-side arithmetic only).

FLOP convention: the forward pass does two N x N x d products per head, 4 N^2 d
FLOPs ("FlashAttention and online softmax", ML Systems Lesson 4, section 3 'HBM
traffic', roofline paragraph); the backward pass does five, 10 N^2 d ("Backward
pass: recompute instead of store", FLOPs paragraph), i.e. 2.5x the forward.  A
causal mask halves both (section "Causal masks and FlashAttention-3").

Byte convention (algorithmic HBM bytes, what the method itself must move): the
forward reads Q, K, V and writes O plus one fp32 lse per row; the backward reads
Q, K, V, O, dO, lse and writes dQ, dK, dV plus one fp32 D per row (which it then
reads back).  Re-reads of K/V by different query tiles are not counted: they are
the cacheable part of the traffic formula 2Nd + 2N^2 d / Br of section 'HBM
traffic'.
"""
from __future__ import annotations

__all__ = [
    "fwd_flops", "bwd_flops", "fwd_bytes", "bwd_bytes", "standard_traffic_elems",
    "flash_traffic_elems", "causal_tiles", "MI355X_BF16_DENSE_PEAK_TFLOPS",
    "MI355X_HBM_PEAK_GBS", "elem_bytes",
]

# MI355X published dense peaks used as roofline denominators.
MI355X_BF16_DENSE_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA (2.5 PFLOP/s)
MI355X_FP32_MFMA_PEAK_TFLOPS = 157.3
MI355X_HBM_PEAK_GBS = 8000.0             # 8 TB/s HBM3E


def elem_bytes(dtype: str) -> int:
    return {"bf16": 2, "fp32": 4}[dtype]


def fwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    return 2.5 * fwd_flops(B, H, N, d, causal)


def fwd_bytes(B: int, H: int, N: int, d: int, dtype: str) -> int:
    s = elem_bytes(dtype)
    return 4 * B * H * N * d * s + 4 * B * H * N


def bwd_bytes(B: int, H: int, N: int, d: int, dtype: str) -> int:
    s = elem_bytes(dtype)
    # read Q, K, V, O, dO; write dQ, dK, dV; lse read, D written then read
    return 8 * B * H * N * d * s + 12 * B * H * N


def standard_traffic_elems(N: int, d: int) -> int:
    """HBM elements of standard attention per head: 4N^2 + 4Nd."""
    return 4 * N * N + 4 * N * d


def flash_traffic_elems(N: int, d: int, Br: int) -> float:
    """HBM elements of the tiled forward per head, no cache: 2Nd + 2N^2 d / Br."""
    return 2 * N * d + 2 * N * N * d / Br


def causal_tiles(N: int, Bt: int) -> tuple[int, int]:
    """(computed, total) square tiles of a causal N x N score matrix cut in Bt x Bt tiles."""
    T = -(-N // Bt)
    return T * (T + 1) // 2, T * T


def splitkv_blocks(B: int, H: int, num_splits: int) -> int:
    """Workgroups of a split-KV decoding pass: one per (batch, head, chunk)
    ("Split-KV for decoding (flash-decoding)")."""
    return B * H * num_splits


def splitkv_bytes(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, num_splits: int) -> dict:
    """Algorithmic HBM bytes of split-KV decoding: the partial pass reads Q, K, V and
    writes fp32 (o, lse) partials; the merge reads the partials and writes O, lse."""
    e = elem_bytes(dtype)
    part = num_splits * B * H * Nq * (d + 1) * 4
    return {"partial": B * H * (Nq + 2 * Nk) * d * e + part,
            "merge": part + B * H * Nq * (d * e + 4)}


def window_pairs(N: int, window: int) -> int:
    """Visible (query, key) pairs of an N-row causal band of width W (all of the
    causal triangle for W <= 0): sum over i of min(i + 1, W)."""
    if window <= 0 or window >= N:
        return N * (N + 1) // 2
    return window * (window + 1) // 2 + (N - window) * window


def varlen_pairs(lengths, causal: bool, window: int = 0) -> int:
    """Visible pairs of a packed batch: each sequence attends only within itself."""
    tot = 0
    for n in lengths:
        n = int(n)
        tot += window_pairs(n, window) if causal else n * n
    return tot
