"""Pins for oracle.kvcache: the after-image of an append is the before-image
with exactly the mapped slots replaced (checked against numpy fancy
assignment and against the slot-by-slot definition), and negative slots store
nothing."""
import numpy as np

from oracle import kvcache as K


def test_append_matches_fancy_assignment():
    rng = np.random.default_rng(0)
    before = rng.integers(0, 2**16, size=(64, 3, 8), dtype=np.uint16)
    slots = rng.permutation(64)[:20]
    rows = rng.integers(0, 2**16, size=(20, 3, 8), dtype=np.uint16)
    want = before.copy()
    want[slots] = rows
    got = K.append_expected(before, rows, slots)
    assert np.array_equal(got, want)
    untouched = np.setdiff1d(np.arange(64), slots)
    assert np.array_equal(got[untouched], before[untouched])


def test_negative_slots_store_nothing():
    before = np.zeros((4, 2), dtype=np.uint16)
    rows = np.ones((3, 2), dtype=np.uint16)
    got = K.append_expected(before, rows, [-1, 2, -5])
    assert got.tolist() == [[0, 0], [0, 0], [1, 1], [0, 0]]
