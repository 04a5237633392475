"""Pins of the oracle's router step (softmax -> top-k with ties to the lower id -> renorm)."""

import numpy as np
import pytest

from oracle.moe import router_topk


def test_equal_logits_pick_the_lowest_ids():
    # a row of equal logits: every probability is 1/E, ties go to the lower id
    lg = np.full((3, 10), 0.75, dtype=np.float32)
    idx, w = router_topk(lg, 4, renorm=False)
    assert (idx == np.arange(4)).all()
    assert np.allclose(w, 0.1, rtol=0, atol=1e-15)
    idx, w = router_topk(lg, 4, renorm=True)
    assert np.allclose(w, 0.25, rtol=0, atol=1e-15)


def test_monotone_rows():
    E = 9
    up = np.arange(E, dtype=np.float32)[None, :]
    idx, _ = router_topk(up, 3, renorm=False)
    assert list(idx[0]) == [8, 7, 6]
    idx, _ = router_topk(-up, 3, renorm=False)
    assert list(idx[0]) == [0, 1, 2]


def test_matches_a_sort_by_logit_then_id():
    # probability order is logit order (softmax is increasing): compare with a library
    # lexicographic sort on (-logit, id), including planted ties
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 33)).astype(np.float32)
    lg[:, 7] = lg[:, 20]          # ties between ids 7 and 20
    lg[5, :] = lg[5, 0]           # a row of ties
    idx, w = router_topk(lg, 6, renorm=False)
    for t in range(lg.shape[0]):
        order = np.lexsort((np.arange(33), -lg[t].astype(np.float64)))[:6]
        assert list(idx[t]) == list(order)
        p = np.exp(lg[t].astype(np.float64) - lg[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[order], rtol=1e-15, atol=0)


def test_softmax_closed_forms():
    # two experts, logits (a, b): p = sigmoid(a - b); shift invariance; renorm sums to 1
    lg = np.array([[2.0, -1.0], [-1.0, 2.0]], dtype=np.float32)
    idx, w = router_topk(lg, 1, renorm=False)
    assert list(idx[:, 0]) == [0, 1]
    assert np.allclose(w[:, 0], 1 / (1 + np.exp(-3.0)), rtol=1e-15)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 12))                 # fp64: the shift below is exact
    i1, w1 = router_topk(x, 5, renorm=False)
    i2, w2 = router_topk(x + 3.5, 5, renorm=False)
    assert (i1 == i2).all() and np.allclose(w1, w2, rtol=1e-12)
    _, wr = router_topk(x, 5, renorm=True)
    assert np.allclose(wr.sum(axis=1), 1.0, rtol=1e-15)
    assert np.allclose(wr, w1 / w1.sum(axis=1, keepdims=True), rtol=1e-15)


def test_masked_experts_and_bad_k():
    # -inf logits have probability 0 and are chosen last (in id order)
    lg = np.array([[-np.inf, 1.0, -np.inf, 0.0]], dtype=np.float32)
    idx, w = router_topk(lg, 3, renorm=False)
    assert list(idx[0]) == [1, 3, 0]
    assert w[0, 2] == 0.0
    with pytest.raises(ValueError):
        router_topk(lg, 5, renorm=False)
