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
* ``tiled_forward`` is the tiled forward pass of "The online softmax theorem /
  The tiled forward pass" (query tile kept, K/V tiles streamed, causal tiles above
  the diagonal skipped as in "Causal masks and FlashAttention-3").  It is the
  method's schedule, used to show that the schedule reaches the oracle's result.
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


def tiled_forward(Q, K, V, scale: float, Br: int = 16, Bc: int = 16, causal: bool = False):
    """Tiled forward pass for one head (Q, K, V: [N, d]); returns (O, lse).

    Per query tile: m = -inf, l = 0, acc = 0; for each K/V tile (skipping tiles that
    lie wholly above the causal diagonal) compute the score tile, update m, rescale
    l and acc by exp(m_old - m_new), add the tile's terms; divide once at the end.
    """
    Q, K, V = (np.asarray(t, dtype=np.float64) for t in (Q, K, V))
    N, d = Q.shape
    O, lse = np.zeros_like(Q), np.empty(N)
    for i in range(0, N, Br):
        q = Q[i:i + Br]
        r = q.shape[0]
        m, l, acc = np.full(r, -np.inf), np.zeros(r), np.zeros((r, d))
        for j in range(0, N, Bc):
            if causal and j > i + r - 1:
                break
            s = scale * (q @ K[j:j + Bc].T)
            if causal:
                rows = np.arange(i, i + r)[:, None]
                cols = np.arange(j, j + s.shape[1])[None, :]
                s = np.where(cols <= rows, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            live = m_new > -np.inf
            m_ref = np.where(live, m_new, 0.0)
            f = np.where(m == -np.inf, 0.0, np.exp(np.where(live, m, 0.0) - m_ref))
            p = np.exp(s - m_ref[:, None])
            p[~live] = 0.0
            l = f * l + p.sum(axis=1)
            acc = f[:, None] * acc + p @ V[j:j + Bc]
            m = m_new
        O[i:i + r] = acc / l[:, None]
        lse[i:i + r] = m + np.log(l)
    return O, lse
