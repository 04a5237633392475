"""Pins of the oracle's routing bookkeeping: library routines, invariants, a hand example."""

import numpy as np
import pytest

from oracle.moe import route


def _check_against_library(idx, E):
    counts, offsets, perm, inv = route(idx, E)
    flat = idx.reshape(-1)
    A = flat.size
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(inv[perm], np.arange(A))
    assert counts.sum() == A and offsets[E] == A
    assert (np.diff(offsets) >= 0).all()
    # every position p holds a slot whose expert owns that position
    owner = np.repeat(np.arange(E), counts)
    assert np.array_equal(flat[perm], owner)


def test_route_hand_example():
    idx = np.array([[2, 0], [0, 2], [1, 2]], dtype=np.int32)
    counts, offsets, perm, inv = route(idx, 4)
    assert counts.tolist() == [2, 1, 3, 0]
    assert offsets.tolist() == [0, 2, 3, 6, 6]
    assert perm.tolist() == [1, 2, 4, 0, 3, 5]
    assert inv.tolist() == [3, 0, 1, 4, 2, 5]


@pytest.mark.parametrize("T,k,E,seed", [(32, 2, 8, 0), (4096, 4, 60, 1), (16, 4, 60, 2),
                                        (8192, 8, 256, 3), (1, 1, 1, 4), (7, 3, 3, 5)])
def test_route_matches_library(T, k, E, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    _check_against_library(idx, E)


def test_route_skewed_and_empty_experts():
    rng = np.random.default_rng(7)
    idx = np.where(rng.random((500, 8)) < 0.9, 5, rng.integers(0, 256, (500, 8))).astype(np.int32)
    _check_against_library(idx, 256)
    idx1 = np.full((64, 4), 3, dtype=np.int32)      # every slot on one expert
    counts, offsets, perm, inv = route(idx1, 60)
    assert counts[3] == 256 and counts.sum() == 256
    assert perm.tolist() == list(range(256))


def test_route_empty_input():
    counts, offsets, perm, inv = route(np.zeros((0, 4), dtype=np.int32), 10)
    assert counts.sum() == 0 and offsets.tolist() == [0] * 11 and perm.size == 0


def test_route_rejects_out_of_range():
    with pytest.raises(IndexError):
        route(np.array([[0, 4]]), 4)
    with pytest.raises(IndexError):
        route(np.array([[-1, 0]]), 4)
