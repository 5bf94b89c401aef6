"""CPU fp64 oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module: only
the tests, the smoke check and the CPU-baseline leg of the benchmark call it.  It
shares no code with the HIP kernels.

What it computes is the plain definition, written out without tiling, blocking of
the softmax or reordering:

* Forward -- "FlashAttention and online softmax" (ML Systems, Lesson 4), section
  "2. The picture / The GPU picture: keep the tile on chip": O = softmax(tau Q K^T) V
  with the softmax taken row by row, and the per-row logsumexp
  lse_i = log sum_j exp(S_ij) (natural log; section "3 / The online softmax
  theorem" gives m_T + log l_T = lse).  The safe softmax subtracts the row max
  before exponentiating (section "One query, one pass").
* Causal mask -- same page, section "Causal masks and FlashAttention-3": query i
  sees key j only when j <= i (the "5. In code" listing builds it with a lower
  triangle).
* Backward -- same page, section "Backward pass: recompute instead of store":
  dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P o (dP - D),
  dQ = tau dS K, dK = tau dS^T Q.  The oracle forms D from P and dP; the identity
  D_i = dO_i . O_i is something the tests check, not something used here.
* Fully masked rows -- same page, "Merging two partial results" and "7. Common
  mistakes": an empty key set has lse = -inf and contributes nothing; a row with no
  visible key returns o = 0, lse = -inf, and no -inf - (-inf) is ever evaluated.

Everything is float64.  Inputs are taken as given (the caller passes exactly the
values the GPU receives, e.g. bf16-rounded values upcast to float64).  For long
sequences the query rows are processed in blocks of ``row_block`` rows; each block
still materialises complete rows of S, P and dP, so every softmax is taken over its
full row -- this bounds memory, it does not change the arithmetic.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_fwd", "attention_bwd", "visible_mask"]


def visible_mask(n_q: int, n_k: int, causal: bool, q_offset: int = 0) -> np.ndarray | None:
    """Boolean (n_q, n_k) table of visible (query, key) pairs, or None if all visible.

    Causal convention (Lesson 4, "Causal masks and FlashAttention-3"): query i sees
    key j iff j <= i.  ``q_offset`` is the absolute index of the first query row.
    """
    if not causal:
        return None
    rows = np.arange(q_offset, q_offset + n_q)[:, None]
    cols = np.arange(n_k)[None, :]
    return cols <= rows


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _rows_softmax(S: np.ndarray, vis: np.ndarray | None):
    """Safe softmax of full rows: returns (P, lse).

    m_i = max over visible j of S_ij; l_i = sum_j exp(S_ij - m_i); lse_i = m_i + ln l_i;
    P_ij = exp(S_ij - m_i) / l_i on visible entries and 0 elsewhere (equal to
    exp(S_ij - lse_i), but without the rounding of lse at large |S|).  Rows with no
    visible entry get P = 0 and lse = -inf (no -inf - (-inf) is formed).
    """
    if vis is not None:
        S = np.where(vis, S, -np.inf)
    m = S.max(axis=1)
    empty = ~np.isfinite(m)  # only -inf can occur: a row with no visible key
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])  # exponents <= 0 on visible entries, exp(-inf)=0
    l = E.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    P = E / l_safe[:, None]  # softmax = exp(S - m) / l; empty rows stay all zero
    return P, lse


def _check_shapes(Q, K, V):
    if Q.ndim != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must all be [B, H, N, d] with the same shape")


def attention_fwd(Q, K, V, scale: float, causal: bool = False, mask=None,
                  row_block: int = 2048):
    """Naive attention forward on [B, H, N, d] arrays.

    Returns (O, lse): O is [B, H, N, d] float64, lse is [B, H, N] float64 (natural
    log, scale included).  ``mask`` (optional, boolean [N, N], True = visible) is
    combined with the causal rule; it exists so tests can reach fully masked rows.
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    _check_shapes(Q, K, V)
    B, H, N, d = Q.shape
    O = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            q, k, v = Q[b, h], K[b, h], V[b, h]
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                S = scale * (q[r0:r1] @ k.T)  # full rows r0..r1 of the N x N scores
                vis = visible_mask(r1 - r0, N, causal, r0)
                if mask is not None:
                    m_rows = np.asarray(mask, dtype=bool)[r0:r1]
                    vis = m_rows if vis is None else (vis & m_rows)
                P, l = _rows_softmax(S, vis)
                O[b, h, r0:r1] = P @ v
                lse[b, h, r0:r1] = l
    return O, lse


def attention_bwd(Q, K, V, dO, scale: float, causal: bool = False, mask=None,
                  row_block: int = 2048, return_D: bool = False):
    """Analytic backward of attention: gradients of sum(dO * O) w.r.t. Q, K, V.

    Recomputes S and P from Q and K (full rows), then
    dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P o (dP - D),
    dQ = scale * dS K, dK = scale * dS^T Q.
    Returns (dQ, dK, dV) [, D] as float64.
    """
    Q, K, V, dO = _as64(Q), _as64(K), _as64(V), _as64(dO)
    _check_shapes(Q, K, V)
    if dO.shape != Q.shape:
        raise ValueError("dO must have the shape of Q")
    B, H, N, d = Q.shape
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    Dall = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            q, k, v, do = Q[b, h], K[b, h], V[b, h], dO[b, h]
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                S = scale * (q[r0:r1] @ k.T)
                vis = visible_mask(r1 - r0, N, causal, r0)
                if mask is not None:
                    m_rows = np.asarray(mask, dtype=bool)[r0:r1]
                    vis = m_rows if vis is None else (vis & m_rows)
                P, _ = _rows_softmax(S, vis)
                dV[b, h] += P.T @ do[r0:r1]
                dP = do[r0:r1] @ v.T
                D = (P * dP).sum(axis=1)
                dS = P * (dP - D[:, None])
                dQ[b, h, r0:r1] = scale * (dS @ k)
                dK[b, h] += scale * (dS.T @ q[r0:r1])
                Dall[b, h, r0:r1] = D
    if return_D:
        return dQ, dK, dV, Dall
    return dQ, dK, dV
