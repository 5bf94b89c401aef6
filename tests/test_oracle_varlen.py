"""Pins of oracle/varlen.py: variable-length batches and the causal sliding window.

Pages: "FlashAttention from Scratch" ("Pitfalls that turn into incidents":
cu_seqlens instead of padding); "FlashAttention and online softmax" (Lesson 4),
"Where it shows up" (sliding-window masks with tile skipping) and "Causal masks and
FlashAttention-3" (8,256 of 16,384 tiles at N = 16384 with 128-tiles).
"""
import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import attention_bwd, attention_fwd
from oracle.varlen import varlen_bwd, varlen_fwd, window_mask, window_tiles


def _r(rng, *s):
    return rng.standard_normal(s)


def test_window_one_is_the_diagonal():
    """W = 1: each query sees only its own key, so o_i = v_i and lse_i = s_ii."""
    rng = np.random.default_rng(0)
    Q, K, V = (_r(rng, 1, 2, 9, 4) for _ in range(3))
    O, lse = attention_fwd(Q, K, V, 0.5, True, mask=window_mask(9, 1))
    np.testing.assert_allclose(O, V, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bhnd,bhnd->bhn", Q, K), rtol=0, atol=1e-14)


def test_window_two_closed_form():
    """W = 2: row i >= 1 is the two-term softmax of keys i-1 and i."""
    rng = np.random.default_rng(1)
    Q, K, V = (_r(rng, 1, 1, 6, 3) for _ in range(3))
    O, lse = attention_fwd(Q, K, V, 1.0, True, mask=window_mask(6, 2))
    q, k, v = Q[0, 0], K[0, 0], V[0, 0]
    for i in range(1, 6):
        a, b = q[i] @ k[i - 1], q[i] @ k[i]
        l = np.log(np.exp(a) + np.exp(b))
        assert abs(lse[0, 0, i] - l) < 1e-14
        np.testing.assert_allclose(O[0, 0, i], np.exp(a - l) * v[i - 1] + np.exp(b - l) * v[i],
                                   rtol=0, atol=1e-14)


@pytest.mark.parametrize("w", [3, 7])
def test_window_rows_by_hand(w):
    rng = np.random.default_rng(w)
    n, scale = 12, 0.8
    Q, K, V = (_r(rng, 1, 1, n, 4) for _ in range(3))
    O, lse = attention_fwd(Q, K, V, scale, True, mask=window_mask(n, w))
    for i in range(n):
        keys = [j for j in range(n) if i - w < j <= i]
        s = [scale * float(Q[0, 0, i] @ K[0, 0, j]) for j in keys]
        L = logsumexp(s)
        assert abs(lse[0, 0, i] - L) < 1e-13
        ref = sum(np.exp(sj - L) * V[0, 0, j] for sj, j in zip(s, keys))
        np.testing.assert_allclose(O[0, 0, i], ref, rtol=0, atol=1e-13)


def test_wide_window_is_causal():
    rng = np.random.default_rng(4)
    Q, K, V = (_r(rng, 1, 1, 20, 4) for _ in range(3))
    a = attention_fwd(Q, K, V, 0.3, True, mask=window_mask(20, 20))
    b = attention_fwd(Q, K, V, 0.3, True)
    np.testing.assert_array_equal(a[0], b[0])
    assert window_mask(20, 0) is None


def test_tile_count_causal_matches_the_pages():
    """Lesson 4, causal masks: N = 16384 in 128-tiles is 16,384 tiles, 8,256 visited."""
    assert window_tiles(16384, 128, 0) == 8256
    assert window_tiles(16384, 128, 16384) == 8256


@pytest.mark.parametrize("n,t,w", [(1024, 64, 256), (16384, 128, 4096), (1000, 32, 96), (512, 128, 128)])
def test_tile_count_closed_form(n, t, w):
    """For W a multiple of the tile and n of the tile: query tile qi visits key tiles
    qi - W/t .. qi, clipped at 0, i.e. min(qi + 1, W/t + 1) of them."""
    T = -(-n // t)
    if n % t == 0 and w % t == 0:
        assert window_tiles(n, t, w) == sum(min(qi + 1, w // t + 1) for qi in range(T))
    assert window_tiles(n, t, w) <= T * (T + 1) // 2


def _dense_to_packed(x):
    B, H, N, d = x.shape
    return np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(H, B * N, d))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5)])
def test_varlen_equal_lengths_is_dense(causal, window):
    rng = np.random.default_rng(5)
    B, H, N, d = 3, 2, 11, 4
    Q, K, V, dO = (_r(rng, B, H, N, d) for _ in range(4))
    cu = np.arange(B + 1) * N
    m = window_mask(N, window)
    O, lse = attention_fwd(Q, K, V, 0.6, causal, mask=m)
    Ov, lv = varlen_fwd(*(_dense_to_packed(x) for x in (Q, K, V)), cu, 0.6, causal, window)
    np.testing.assert_allclose(Ov, _dense_to_packed(O), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lv, lse.transpose(1, 0, 2).reshape(H, B * N), rtol=0, atol=1e-14)
    g = attention_bwd(Q, K, V, dO, 0.6, causal, mask=m)
    gv = varlen_bwd(*(_dense_to_packed(x) for x in (Q, K, V, dO)), cu, 0.6, causal, window)
    for a, b in zip(gv, g):
        np.testing.assert_allclose(a, _dense_to_packed(b), rtol=0, atol=1e-13)


def test_varlen_sequences_are_independent():
    """Changing one sequence's inputs leaves every other sequence's outputs unchanged,
    and an empty sequence is allowed."""
    rng = np.random.default_rng(6)
    cu = np.array([0, 5, 5, 17, 20])
    Q, K, V = (_r(rng, 2, 20, 4) for _ in range(3))
    O1, l1 = varlen_fwd(Q, K, V, cu, 0.5, True)
    K2 = K.copy()
    K2[:, 5:17] += _r(rng, 2, 12, 4)  # sequence 2 only (a row-constant shift would cancel)
    O2, l2 = varlen_fwd(Q, K2, V, cu, 0.5, True)
    other = np.r_[0:5, 17:20]
    np.testing.assert_array_equal(O1[:, other], O2[:, other])
    np.testing.assert_array_equal(l1[:, other], l2[:, other])
    assert np.abs(O1[:, 5:17] - O2[:, 5:17]).max() > 1e-3
