"""Pins for oracle.residency: pick counts, decayed scores, the swap rule with
its hysteresis, the pool moves, and the fingerprint of the byte audit.

Against: SplitMix64's published outputs (tests/golden/splitmix64.txt) for the
fingerprint, hand-worked swap examples, and invariants (pool sizes, the
stable state the rule reaches, no swap back inside the hysteresis band,
bytes found again at their new homes)."""
import os

import numpy as np
import pytest

from oracle import residency as res
from tests import brute


def _golden():
    out = {}
    with open(os.path.join(brute.GOLDEN, "splitmix64.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                seed, n, v = (int(t) for t in line.split())
                out[(seed, n)] = v
    return out


def test_fingerprint_matches_published_splitmix64():
    g = _golden()
    for seed in (0, 1234567):
        n_max = max(n for s, n in g if s == seed)
        for n in range(1, n_max + 1):
            # mix64(seed + n * gamma) is the generator's n-th output
            z = np.uint64((seed + n * res.GOLDEN_GAMMA) % 2**64)
            assert int(res.mix64(z)) == g[(seed, n)]
            # a blob of n words all equal to the seed fingerprints to the sum of the first n outputs
            blob = np.full(n, seed, dtype="<u8").view(np.uint8)
            assert res.fingerprint(blob) == sum(g[(seed, m)] for m in range(1, n + 1)) % 2**64


def test_fingerprint_sees_every_change(rng):
    blob = rng.integers(0, 256, 4096, dtype=np.uint8)
    fp = res.fingerprint(blob)
    for _ in range(200):
        b = blob.copy()
        i, bit = int(rng.integers(0, blob.size)), int(rng.integers(0, 8))
        b[i] ^= np.uint8(1 << bit)
        assert res.fingerprint(b) != fp
    w = blob.view("<u8").copy()
    w[[3, 7]] = w[[7, 3]]                      # two words exchanged
    assert res.fingerprint(w.view(np.uint8)) != fp
    assert res.fingerprint(np.roll(blob, 8)) != fp   # the same words one position later
    with pytest.raises(ValueError):
        res.fingerprint(blob[:12])


def test_count_picks():
    ids = np.array([[0, 3], [3, 5], [7, -1], [9, 3]], dtype=np.int32)   # -1 and 9 out of range (E=8)
    assert res.count_picks(ids, 8).tolist() == [1, 0, 0, 3, 0, 1, 0, 1]


def test_update_scores():
    s = res.update_scores([4.0, 1.0, 0.0], [1, 0, 3], 0.5)
    assert s.tolist() == [3.0, 0.5, 3.0]


SLOT8 = np.array([0, 1, 2, 3, 4, -1, -2, -3], dtype=np.int32)   # 0-4 hot, 5-7 cold
SCORE8 = np.array([5.0, 0.5, 2.0, 0.0, 9.0, 10.0, 1.4, 3.0])


def test_plan_hand_worked():
    # threshold 3: 10 > 3*max(0, 1) swaps 5 for 3; 3 > 3*max(0.5, 1) is false: stop
    pairs, slot = res.plan_swaps(SLOT8, SCORE8, 3.0, 1.0, 64)
    assert pairs == [(5, 3)]
    assert slot.tolist() == [0, 1, 2, -1, 4, 3, -2, -3]
    # threshold 1.5: also 3 > 1.5 swaps 7 for 1; then 1.4 > 1.5*2 is false
    pairs, slot = res.plan_swaps(SLOT8, SCORE8, 1.5, 1.0, 64)
    assert pairs == [(5, 3), (7, 1)]
    assert slot.tolist() == [0, -3, 2, -1, 4, 3, -2, 1]
    # at most one swap
    assert res.plan_swaps(SLOT8, SCORE8, 1.5, 1.0, 1)[0] == [(5, 3)]
    # min_score: a never-picked hot expert still needs min_score*threshold
    assert res.plan_swaps(SLOT8, SCORE8, 3.0, 4.0, 64)[0] == []


def test_plan_ties_go_to_the_lower_index():
    slot = np.array([0, 1, -1, -2], dtype=np.int32)
    score = np.array([1.0, 1.0, 7.0, 7.0])
    pairs, _ = res.plan_swaps(slot, score, 3.0, 1.0, 1)
    assert pairs == [(2, 0)]
    pairs, _ = res.plan_swaps(slot, score, 3.0, 1.0, 8)
    assert pairs == [(2, 0), (3, 1)]


@pytest.mark.parametrize("threshold", [1.0, 1.5, 3.0])
def test_plan_reaches_a_stable_table(rng, threshold):
    for _ in range(50):
        E, n_hot = 24, int(rng.integers(1, 23))
        hot = set(rng.choice(E, n_hot, replace=False).tolist())
        slot = np.empty(E, dtype=np.int32)
        h = c = 0
        for e in range(E):
            if e in hot:
                slot[e], h = h, h + 1
            else:
                slot[e], c = -c - 1, c + 1
        score = rng.exponential(3.0, E) * (rng.random(E) < 0.8)
        pairs, new = res.plan_swaps(slot, score, threshold, 1.0, 10**6)
        # pools keep their sizes and every slot index appears once
        assert sorted(new[new >= 0].tolist()) == list(range(n_hot))
        assert sorted((-new[new < 0] - 1).tolist()) == list(range(E - n_hot))
        # every pair moved one cold expert in and one hot expert out
        for cc, hh in pairs:
            assert slot[cc] < 0 <= slot[hh] and new[cc] == slot[hh] and new[hh] == slot[cc]
        # nothing left that the rule would still swap
        cold_max = max((score[e] for e in range(E) if new[e] < 0), default=-np.inf)
        hot_min = min(score[e] for e in range(E) if new[e] >= 0)
        assert not cold_max > threshold * max(hot_min, 1.0)
        assert res.plan_swaps(new, score, threshold, 1.0, 10**6)[0] == []


def test_hysteresis_blocks_the_swap_back():
    slot = np.array([0, 1, -1, -2], dtype=np.int32)            # 0, 1 hot; 2, 3 cold
    pairs, slot, score = res.manager_tick(slot, np.zeros(4), [1, 9, 10, 0], 1.0, 3.0, 1.0, 64)
    assert pairs == [(2, 0)] and slot.tolist() == [-1, 1, 0, -2]
    # expert 0 (now cold) is picked twice as often as 2, which replaced it:
    # decayed scores settle at 2x the per-tick counts (16 against 8), inside
    # the band (16 <= 3 * 8), so 0 stays out; with no band it would come back
    for _ in range(40):
        pairs, slot, score = res.manager_tick(slot, score, [8, 20, 4, 0], 0.5, 3.0, 1.0, 64)
        assert pairs == []
    assert res.plan_swaps(slot, score, 1.0, 1.0, 64)[0] == [(0, 2)]
    # picked ten times as often, it comes back
    back = []
    for _ in range(10):
        pairs, slot, score = res.manager_tick(slot, score, [40, 20, 4, 0], 0.5, 3.0, 1.0, 64)
        back += pairs
    assert back == [(0, 2)] and slot.tolist() == [0, 1, -1, -2]


def test_moves_keep_every_expert_intact(rng):
    E, B = 8, 64
    blobs = rng.integers(0, 256, (E, B), dtype=np.uint8)
    slot = SLOT8.copy()
    hot_pool = np.stack([blobs[e] for e in range(E) if slot[e] >= 0])
    host_pool = np.stack([blobs[e] for e in range(E) if slot[e] < 0])
    boot = [res.fingerprint(blobs[e]) for e in range(E)]
    for threshold in (1.5, 1.0):
        pairs, new = res.plan_swaps(slot, SCORE8, threshold, 1.0, 64)
        hot_pool, host_pool = res.apply_swaps(slot, pairs, hot_pool, host_pool)
        slot = new
        for e in range(E):
            home = hot_pool[slot[e]] if slot[e] >= 0 else host_pool[-slot[e] - 1]
            assert np.array_equal(home, blobs[e])
            assert res.fingerprint(home) == boot[e]
