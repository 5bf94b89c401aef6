"""CPU fp64 oracle for split-KV attention (decoding) and the merge of partials.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module: only
the tests, the smoke check and the CPU-baseline leg of the benchmark call it.  It
shares no code with the HIP kernels.

Source: "FlashAttention and online softmax" (ML Systems, Lesson 4):

* section "Split-KV for decoding (flash-decoding)": the keys of each query row
  are cut into k chunks, each chunk returns a partial (o, lse) over its keys alone,
  and a second step merges the k partials of a row;
* section "Merging two partial results": for disjoint key sets A and B with
  normalised outputs o_A, o_B and logsumexps lse_A, lse_B, the union has
  lse = log(e^lse_A + e^lse_B) and o = e^(lse_A - lse) o_A + e^(lse_B - lse) o_B;
  an empty set has lse = -inf and weight 0, and two empty sets give o = 0,
  lse = -inf.  The merge is associative, so k partials fold in any order.

Reading of the causal rule when a row block of Nq queries attends to Nk >= Nq
keys (the pages state it only for square attention, "j <= i"): the queries are
the last Nq positions of the sequence, so query i (0-based among the Nq) sees key
j iff j <= i + (Nk - Nq).  For Nq = Nk this is the square rule; for one decoding
query it makes every key visible.

Split rule (the library states the same one): with c = ceil(Nk / k), split s
covers keys [s*c, min(Nk, (s+1)*c)); splits that start at or past Nk are empty.
"""
from __future__ import annotations

import numpy as np

from .online import merge

__all__ = ["visible_rect", "attention_fwd_rect", "split_ranges", "splitkv_partials",
           "merge_partials"]


def visible_rect(n_q: int, n_k: int, causal: bool) -> np.ndarray | None:
    """(n_q, n_k) table of visible pairs, or None when every key is visible."""
    if not causal:
        return None
    rows = np.arange(n_q)[:, None] + (n_k - n_q)
    cols = np.arange(n_k)[None, :]
    return cols <= rows


def _softmax_rows(S: np.ndarray, vis: np.ndarray | None):
    """Safe softmax of complete rows: (P, lse); rows with no visible key give P = 0,
    lse = -inf.  Written out here rather than shared with attention.py so that each
    oracle module reads on its own."""
    if vis is not None:
        S = np.where(vis, S, -np.inf)
    m = S.max(axis=1)
    empty = ~np.isfinite(m)
    m0 = np.where(empty, 0.0, m)
    E = np.exp(S - m0[:, None])
    l = E.sum(axis=1)
    l1 = np.where(empty, 1.0, l)
    lse = np.where(empty, -np.inf, m0 + np.log(l1))
    return E / l1[:, None], lse


def attention_fwd_rect(Q, K, V, scale: float, causal: bool = False, key_range=None):
    """Plain attention of Q [B,H,Nq,d] over K, V [B,H,Nk,d].

    ``key_range`` = (begin, end) restricts every row to keys begin <= j < end
    (intersected with the causal rule); the softmax is then over that set alone.
    Returns O [B,H,Nq,d] and lse [B,H,Nq] in float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    if K.shape != (B, H, n_k, d) or V.shape != K.shape:
        raise ValueError("K and V must be [B, H, Nk, d] with Q's B, H, d")
    vis = visible_rect(n_q, n_k, causal)
    if key_range is not None:
        b0, b1 = key_range
        cols = np.arange(n_k)[None, :]
        rng = np.broadcast_to((cols >= b0) & (cols < b1), (n_q, n_k))
        vis = rng if vis is None else (vis & rng)
    O = np.zeros((B, H, n_q, d))
    lse = np.zeros((B, H, n_q))
    for b in range(B):
        for h in range(H):
            P, l = _softmax_rows(scale * (Q[b, h] @ K[b, h].T), vis)
            O[b, h] = P @ V[b, h]
            lse[b, h] = l
    return O, lse


def split_ranges(n_k: int, num_splits: int):
    """Key range [begin, end) of every split (empty ranges have begin >= end)."""
    c = -(-n_k // num_splits)
    return [(s * c, min(n_k, (s + 1) * c)) for s in range(num_splits)]


def splitkv_partials(Q, K, V, scale: float, causal: bool, num_splits: int):
    """Partial (o, lse) of every split: o_part [S,B,H,Nq,d], lse_part [S,B,H,Nq]."""
    outs, lses = [], []
    for b0, b1 in split_ranges(K.shape[2], num_splits):
        o, l = attention_fwd_rect(Q, K, V, scale, causal, key_range=(b0, b1))
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def merge_partials(o_part, lse_part):
    """Fold the pages' two-set merge over the leading (split) axis."""
    o, lse = o_part[0], lse_part[0]
    for s in range(1, o_part.shape[0]):
        o, lse = merge(o, lse, o_part[s], lse_part[s])
    return o, lse
