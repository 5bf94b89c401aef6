"""Pins of the split-KV oracle (oracle/splitkv.py).

Pages: "FlashAttention and online softmax" (ML Systems Lesson 4), sections
"Split-KV for decoding (flash-decoding)" and "Merging two partial results", and
'Check yourself' question 5.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

from exact_io_aware_14_amd.accounting import splitkv_blocks
from oracle import (attention_fwd, attention_fwd_rect, merge, merge_partials, split_ranges,
                    splitkv_partials, visible_mask, visible_rect)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_decode_example_block_counts(golden):
    """'Check yourself' 5: 4*16 = 64 blocks without split, 64*8 = 512 with 8 chunks."""
    g = golden("splitkv_decode_example.json")
    assert splitkv_blocks(g["batch"], g["heads"], 1) == g["blocks_without_split"]
    assert splitkv_blocks(g["batch"], g["heads"], g["chunks"]) == g["blocks_with_split"]
    assert round(g["blocks_with_split"] / g["sms"]) == g["waves_with_split_about"]


@pytest.mark.parametrize("n", [1, 5, 17])
def test_rect_rule_is_square_rule_when_square(n):
    """For Nq = Nk the bottom-aligned rule is the pages' j <= i."""
    assert np.array_equal(visible_rect(n, n, True), visible_mask(n, n, True))
    assert visible_rect(n, n, False) is None


@pytest.mark.parametrize("causal", [False, True])
def test_rect_equals_square_oracle(causal):
    """attention_fwd_rect on square inputs reproduces the pinned square oracle."""
    rng = np.random.default_rng(1)
    Q, K, V = (_rand(rng, 2, 3, 37, 8) for _ in range(3))
    O1, l1 = attention_fwd_rect(Q, K, V, 0.4, causal)
    O2, l2 = attention_fwd(Q, K, V, 0.4, causal)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_rect_brute_force_rows():
    """Each row by hand: visible keys j <= i + (Nk - Nq); lse by scipy's logsumexp,
    o as the exp-weighted average written as a Python loop."""
    rng = np.random.default_rng(2)
    nq, nk, d, scale = 3, 10, 4, 0.7
    Q, K, V = _rand(rng, 1, 1, nq, d), _rand(rng, 1, 1, nk, d), _rand(rng, 1, 1, nk, d)
    O, lse = attention_fwd_rect(Q, K, V, scale, causal=True)
    for i in range(nq):
        keys = list(range(0, i + (nk - nq) + 1))
        s = [scale * float(Q[0, 0, i] @ K[0, 0, j]) for j in keys]
        ref_lse = logsumexp(s)
        ref_o = sum(np.exp(sj - ref_lse) * V[0, 0, j] for sj, j in zip(s, keys))
        assert abs(lse[0, 0, i] - ref_lse) < 1e-13
        np.testing.assert_allclose(O[0, 0, i], ref_o, rtol=0, atol=1e-13)


def test_one_decode_query_sees_every_key():
    """A single decoding query is the newest position: the causal rule hides nothing."""
    rng = np.random.default_rng(3)
    Q, K, V = _rand(rng, 2, 2, 1, 8), _rand(rng, 2, 2, 50, 8), _rand(rng, 2, 2, 50, 8)
    a = attention_fwd_rect(Q, K, V, 0.3, causal=True)
    b = attention_fwd_rect(Q, K, V, 0.3, causal=False)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("nk,splits", [(10, 1), (10, 3), (10, 4), (10, 8), (10, 16), (257, 7), (64, 64)])
def test_split_ranges_partition(nk, splits):
    """The splits cover 0..Nk-1 once, in order, with chunk ceil(Nk/k); the rest are empty."""
    r = split_ranges(nk, splits)
    assert len(r) == splits
    c = -(-nk // splits)
    covered = [j for b0, b1 in r for j in range(b0, b1)]
    assert covered == list(range(nk))
    assert all(b1 - b0 <= c for b0, b1 in r)


@pytest.mark.parametrize("nq,nk,splits,causal", [
    (1, 100, 1, False), (1, 100, 8, False), (1, 100, 8, True), (1, 7, 16, False),
    (4, 60, 5, True), (4, 4, 4, True), (8, 33, 3, False), (2, 300, 13, True)])
def test_splitting_does_not_change_the_answer(nq, nk, splits, causal):
    """Split-KV section: merging the k partials reproduces full attention (here to
    1e-12 in fp64), including splits with no keys and rows whose split is masked."""
    rng = np.random.default_rng(nq * 1000 + nk + splits)
    Q, K, V = _rand(rng, 2, 2, nq, 16), _rand(rng, 2, 2, nk, 16), _rand(rng, 2, 2, nk, 16)
    o_part, lse_part = splitkv_partials(Q, K, V, 0.25, causal, splits)
    assert o_part.shape == (splits, 2, 2, nq, 16) and lse_part.shape == (splits, 2, 2, nq)
    O, lse = merge_partials(o_part, lse_part)
    O_ref, lse_ref = attention_fwd_rect(Q, K, V, 0.25, causal)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_empty_split_is_minus_inf_and_zero():
    """'Merging two partial results': an empty set has lse = -inf, o = 0."""
    rng = np.random.default_rng(5)
    Q, K, V = _rand(rng, 1, 1, 1, 4), _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 3, 4)
    o_part, lse_part = splitkv_partials(Q, K, V, 1.0, False, 8)  # c = 1: splits 3..7 empty
    assert np.all(lse_part[3:] == -np.inf) and np.all(o_part[3:] == 0.0)
    assert np.all(np.isfinite(lse_part[:3]))


def test_merge_order_does_not_matter():
    """The merge is associative: folding the partials in reverse order agrees."""
    rng = np.random.default_rng(6)
    Q, K, V = _rand(rng, 1, 2, 2, 8), _rand(rng, 1, 2, 90, 8), _rand(rng, 1, 2, 90, 8)
    o_part, lse_part = splitkv_partials(Q, K, V, 0.5, False, 9)
    a = merge_partials(o_part, lse_part)
    b = merge_partials(o_part[::-1], lse_part[::-1])
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_plain_average_is_the_common_mistake():
    """The plain average of two partial outputs is not the merged output unless the
    two sets carry equal weight ('Merging two partial results', the wrong line)."""
    rng = np.random.default_rng(7)
    Q = np.ones((1, 1, 1, 4))
    K = np.zeros((1, 1, 20, 4))
    K[..., 10:, :] = 0.5  # scores 0 on the first set, 2 on the second: weights differ
    V = _rand(rng, 1, 1, 20, 4)
    o_part, lse_part = splitkv_partials(Q, K, V, 1.0, False, 2)
    O, _ = merge_partials(o_part, lse_part)
    assert abs(lse_part[0] - lse_part[1]).max() > 0.1
    assert np.abs(O - 0.5 * (o_part[0] + o_part[1])).max() > 1e-3
