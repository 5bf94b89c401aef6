"""CPU fp64 oracle for variable-length batches and sliding-window masks.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module: only
the tests, the smoke check and the CPU-baseline leg of the benchmark call it.  It
shares no code with the HIP kernels.

* Variable-length batches -- "FlashAttention from Scratch", section "Pitfalls that
  turn into incidents" (do not pad a batch of sequences of different lengths; pass
  the boundaries as cu_seqlens) and its "names you will actually type"
  (flash_attn_varlen_func for ragged batches).  Sequence b holds the rows
  cu[b] .. cu[b+1]-1 of every head, and attends only within itself: the result is
  exactly the attention of each sequence taken alone.  Layout read here: packed
  head-major, [H, T, d] with T = cu[B], lse [H, T].
* Sliding window -- "FlashAttention and online softmax" (Lesson 4), section "Where
  it shows up": long-context training uses causal and sliding-window masks, both
  with tile skipping.  Reading: a causal band of W keys, query i sees key j iff
  i - W < j <= i.

Both reduce to the plain definition in ``attention.py`` applied per sequence with
an explicit visibility table, so no new arithmetic is introduced here.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_bwd, attention_fwd

__all__ = ["window_mask", "window_tiles", "varlen_fwd", "varlen_bwd"]


def window_mask(n: int, window: int) -> np.ndarray | None:
    """[n, n] table of pairs inside the band i - W < j (None for W <= 0: no band).
    Combined with the causal rule j <= i by the callers."""
    if window <= 0:
        return None
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return j > i - window


def window_tiles(n: int, tile: int, window: int) -> int:
    """Number of (query tile, key tile) pairs of a tile x tile grid that hold at
    least one pair visible under the causal band: the tiles a kernel that skips
    empty tiles must visit.  Counted by brute force over the tiles."""
    t = -(-n // tile)
    count = 0
    for qi in range(t):
        q_lo, q_hi = qi * tile, min(n, qi * tile + tile) - 1
        for kj in range(t):
            k_lo, k_hi = kj * tile, min(n, kj * tile + tile) - 1
            # some (i, j) with q_lo <= i <= q_hi, k_lo <= j <= k_hi, i - W < j <= i
            if k_lo <= q_hi and (window <= 0 or k_hi > q_lo - window):
                count += 1
    return count


def _seq(x, h, c0, c1):
    return x[h, c0:c1][None, None]


def varlen_fwd(Q, K, V, cu, scale: float, causal: bool, window: int = 0):
    """Q, K, V: [H, T, d]; cu: B+1 boundaries.  Returns O [H, T, d], lse [H, T]."""
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    H, T, d = Q.shape
    O = np.zeros((H, T, d))
    lse = np.zeros((H, T))
    for b in range(len(cu) - 1):
        c0, c1 = int(cu[b]), int(cu[b + 1])
        if c1 == c0:
            continue
        m = window_mask(c1 - c0, window)
        for h in range(H):
            o, l = attention_fwd(_seq(Q, h, c0, c1), _seq(K, h, c0, c1), _seq(V, h, c0, c1),
                                 scale, causal, mask=m)
            O[h, c0:c1] = o[0, 0]
            lse[h, c0:c1] = l[0, 0]
    return O, lse


def varlen_bwd(Q, K, V, dO, cu, scale: float, causal: bool, window: int = 0):
    """Gradients of sum(dO * O) for the packed layout: (dQ, dK, dV), each [H, T, d]."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    H, T, d = Q.shape
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(len(cu) - 1):
        c0, c1 = int(cu[b]), int(cu[b + 1])
        if c1 == c0:
            continue
        m = window_mask(c1 - c0, window)
        for h in range(H):
            g = attention_bwd(_seq(Q, h, c0, c1), _seq(K, h, c0, c1), _seq(V, h, c0, c1),
                              _seq(dO, h, c0, c1), scale, causal, mask=m)
            dQ[h, c0:c1], dK[h, c0:c1], dV[h, c0:c1] = (x[0, 0] for x in g)
    return dQ, dK, dV
