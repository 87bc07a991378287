"""Pins for oracle.gather: the picked-cold set and the scratch copy.

Against: a hand-worked residency table with its expected cold list and
scratch contents, collections.Counter for pick counts, and the generator's
residency-slot writer."""
from collections import Counter

import numpy as np

from oracle import gather
from synth import gen


def test_hand_worked_gather():
    # experts 0..5; hot: 0, 2, 5; cold: 1 -> slot 0, 3 -> slot 1, 4 -> slot 2
    slot = np.array([0, -1, 1, -2, -3, 2], dtype=np.int32)
    ids = np.array([[3, 1], [3, 0], [5, 2]])
    assert gather.picked_cold(ids, slot).tolist() == [1, 3]
    B = 8
    host = np.arange(3 * B, dtype=np.uint8).reshape(3, B) + 1
    scratch = np.full((3, B), 0xEE, dtype=np.uint8)          # sentinel
    out = gather.gather_cold(ids, slot, host, scratch)
    assert np.array_equal(out[0], host[0])                    # expert 1
    assert np.array_equal(out[1], host[1])                    # expert 3 (picked twice, copied once)
    assert np.all(out[2] == 0xEE)                             # expert 4 unpicked: untouched
    assert np.all(scratch == 0xEE)                            # input not modified


def test_no_cold_when_all_hot():
    slot = np.arange(8, dtype=np.int32)
    ids = np.array([[7, 1], [0, 2]])
    assert gather.picked_cold(ids, slot).size == 0


def test_pick_counts_against_counter():
    rng = np.random.default_rng(0)
    ids = rng.integers(0, 40, (32, 6))
    c = Counter(ids.ravel().tolist())
    got = gather.pick_counts(ids, 40)
    assert [c.get(e, 0) for e in range(40)] == got.tolist()


def test_residency_slots_layout():
    slot = gen.residency_slots([5, 0, 3], 6)
    assert slot.tolist() == [0, -1, -2, 1, -3, 2]
    # hot entries are a permutation of 0..n_hot-1, cold of 0..n_cold-1
    hot = sorted(int(s) for s in slot if s >= 0)
    cold = sorted(-int(s) - 1 for s in slot if s < 0)
    assert hot == [0, 1, 2] and cold == [0, 1, 2]
