"""Reference forms of the one-pass (online) softmax, the lse merge and the tiled
forward pass, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY.  These functions pin the oracle in ``attention.py``
against the worked examples printed on the pages and against the method's own
steps; the product path never imports them.

Sources (all on "FlashAttention and online softmax", ML Systems Lesson 4, unless
noted):

* ``online_softmax`` follows the recurrence of the theorem in section
  "3. Definitions and main results / The online softmax theorem": start from
  m = -inf, l = 0, o~ = 0; per block take m_new = max(m, block max), multiply l and
  o~ by exp(m - m_new), add the block's exp(x - m_new) terms; at the end
  o = o~ / l and lse = m + log l.  A block that leaves m at -inf contributes nothing
  (section "7. Common mistakes": guard m = -inf).
* ``three_pass_softmax_average`` is the safe softmax read three times (max, sum,
  weighted sum) from section "2. The picture / One query, one pass".
* ``merge`` is the formula of section "Merging two partial results", in its stable
  form lse = max + log(1 + exp(-|lse_A - lse_B|)), with the empty-set rules stated
  there (lse = -inf has weight 0; both empty gives o = 0, lse = -inf).
* ``tiled_forward`` is the tiled forward pass of "The online softmax theorem"
  (blocks of queries and of keys, a running reference value, denominator and
  numerator per query row, blocks wholly above the causal diagonal skipped as in
  "Causal masks and FlashAttention-3"), run in either loop order of section "HBM
  traffic".  It shows that the block schedule reaches the oracle's result.
"""
from __future__ import annotations

import numpy as np

__all__ = ["online_softmax", "three_pass_softmax_average", "merge", "tiled_forward"]


def online_softmax(x, v=None, block: int = 1, state=None, trace: bool = False):
    """Run the online-softmax recurrence over scores ``x`` in blocks of ``block``.

    ``v`` (optional) holds one value per score (scalar values, shape [n]) or one
    value row per score (shape [n, d]).  ``state`` = (m, l, o~) to continue from.
    Returns dict(m, l, o_tilde, o, lse[, steps]) where ``steps`` lists
    (m, factor, l, o_tilde) after each block.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    if v is None:
        v = np.zeros(n)
    v = np.asarray(v, dtype=np.float64)
    if state is None:
        m, l = -np.inf, 0.0
        o = np.zeros(v.shape[1:]) if v.ndim > 1 else 0.0
    else:
        m, l, o = state
        m, l = float(m), float(l)
        o = np.array(o, dtype=np.float64) if v.ndim > 1 else float(o)
    steps = []
    for j in range(0, n, block):
        xb, vb = x[j:j + block], v[j:j + block]
        m_new = max(m, float(xb.max()))
        if m_new == -np.inf:           # nothing visible yet: state stays empty
            steps.append((m, 1.0, l, o))
            continue
        factor = 0.0 if m == -np.inf else float(np.exp(m - m_new))
        w = np.exp(xb - m_new)          # every exponent <= 0
        l = factor * l + float(w.sum())
        o = factor * o + (w @ vb if vb.ndim > 1 else float((w * vb).sum()))
        m = m_new
        steps.append((m, factor, l, o))
    if l > 0.0:
        out = o / l
        lse = m + np.log(l)
    else:
        out = np.zeros_like(o) if v.ndim > 1 else 0.0
        lse = -np.inf
    res = dict(m=m, l=l, o_tilde=o, o=out, lse=lse)
    if trace:
        res["steps"] = steps
    return res


def three_pass_softmax_average(x, v):
    """Safe softmax average read three times: max, then sum, then weighted sum."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m = x.max()
    l = np.exp(x - m).sum()
    return (np.exp(x - m) @ v) / l


def merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial attention results over disjoint key sets (many rows at once).

    ``o_*`` are normalised outputs ([..., d] or [...]), ``lse_*`` their logsumexps
    ([...]).  Returns (o, lse).
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    hi = np.maximum(la, lb)
    both_empty = hi == -np.inf
    hi_safe = np.where(both_empty, 0.0, hi)
    # |la - lb| is +inf when exactly one side is empty (weight 0 for it); never -inf - -inf
    gap = np.where(both_empty, 0.0, np.abs(np.where(both_empty, 0.0, la) - np.where(both_empty, 0.0, lb)))
    lse = np.where(both_empty, -np.inf, hi_safe + np.log1p(np.exp(-gap)))
    lse_safe = np.where(both_empty, 0.0, lse)
    wa = np.where(la == -np.inf, 0.0, np.exp(np.where(la == -np.inf, 0.0, la) - lse_safe))
    wb = np.where(lb == -np.inf, 0.0, np.exp(np.where(lb == -np.inf, 0.0, lb) - lse_safe))
    wa = np.where(both_empty, 0.0, wa)
    wb = np.where(both_empty, 0.0, wb)
    if o_a.ndim > wa.ndim:
        wa, wb = wa[..., None], wb[..., None]
    return wa * o_a + wb * o_b, lse


class _RowState:
    """Running state of a set of query rows under the online-softmax theorem: the
    reference value ``ref`` each row's weights are measured against (the largest
    score seen so far, -inf before any visible key), the denominator ``den`` (sum of
    the weights) and the numerator ``num`` (weight-times-value sum, [rows, d])."""

    def __init__(self, rows: int, d: int):
        self.ref = np.full(rows, -np.inf)
        self.den = np.zeros(rows)
        self.num = np.zeros((rows, d))

    def fold(self, sel, scores, values):
        """Fold a block of scores (hidden pairs = -inf) of the rows ``sel`` and their
        value rows into the state.  Rows whose block is wholly hidden keep their state
        (the theorem's empty-block case: never -inf - (-inf))."""
        old = self.ref[sel]
        top = scores.max(axis=1)
        seen = top > -np.inf
        new = np.where(seen, np.maximum(old, top), old)
        # weight of the old state under the new reference: 0 if it was empty
        keep = np.zeros_like(old)
        had = old > -np.inf
        keep[had] = np.exp(old[had] - new[had])
        w = np.zeros_like(scores)
        w[seen] = np.exp(scores[seen] - new[seen][:, None])
        self.den[sel] = keep * self.den[sel] + w.sum(axis=1)
        self.num[sel] = keep[:, None] * self.num[sel] + w @ values
        self.ref[sel] = new

    def result(self):
        """(O, lse): O = num / den and lse = ref + log den; empty rows give O = 0,
        lse = -inf."""
        live = self.den > 0.0
        O = np.zeros_like(self.num)
        O[live] = self.num[live] / self.den[live][:, None]
        lse = np.full(self.den.shape, -np.inf)
        lse[live] = self.ref[live] + np.log(self.den[live])
        return O, lse


def _hidden(q_lo: int, nq: int, k_lo: int, nk: int, causal: bool):
    """[nq, nk] boolean table of the pairs the causal rule hides (key index above the
    query index) in the block of queries q_lo.. and keys k_lo..; None if none is."""
    if not causal or k_lo + nk - 1 <= q_lo:
        return None
    first_hidden = np.arange(q_lo, q_lo + nq) + 1 - k_lo  # per row: first hidden column
    return np.arange(nk)[None, :] >= first_hidden[:, None]


def tiled_forward(Q, K, V, scale: float, Br: int = 16, Bc: int = 16, causal: bool = False,
                  order: str = "kv_outer"):
    """Tiled forward pass of one head (Q, K, V: [N, d]) by the online-softmax theorem;
    returns (O, lse).

    ``order="kv_outer"`` is the schedule of the original paper's algorithm as the
    pages describe it (section "HBM traffic": outer loop over K/V blocks, inner loop
    over query blocks, the per-row running state kept for all N rows between visits).
    ``order="q_outer"`` is the FlashAttention-2 schedule of the same section (each
    query block's state finished before the next block starts).  Either way a block
    pair that the causal rule hides entirely is never touched ("Causal masks and
    FlashAttention-3"), and O is divided by the denominator once at the end.
    """
    Q, K, V = (np.asarray(t, dtype=np.float64) for t in (Q, K, V))
    N, d = Q.shape
    q_blocks = [(a, min(Br, N - a)) for a in range(0, N, Br)]
    k_blocks = [(a, min(Bc, N - a)) for a in range(0, N, Bc)]
    if order == "kv_outer":
        pairs = [(qb, kb) for kb in k_blocks for qb in q_blocks]
    elif order == "q_outer":
        pairs = [(qb, kb) for qb in q_blocks for kb in k_blocks]
    else:
        raise ValueError(f"unknown order {order!r}")
    state = _RowState(N, d)
    for (q_lo, nq), (k_lo, nk) in pairs:
        if causal and k_lo > q_lo + nq - 1:
            continue  # every key of the block lies above every query of the block
        block = scale * (Q[q_lo:q_lo + nq] @ K[k_lo:k_lo + nk].T)
        hide = _hidden(q_lo, nq, k_lo, nk, causal)
        if hide is not None:
            block[hide] = -np.inf
        state.fold(slice(q_lo, q_lo + nq), block, V[k_lo:k_lo + nk])
    return state.result()
