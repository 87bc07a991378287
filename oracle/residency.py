"""Adaptive residency and the byte audit (test infrastructure, like all of
oracle/).

The gracetier write-up: between decode steps a manager moves experts that
are being picked often into the hot (HBM) set and moves quiet ones out
(section 1, "The idea"); swapping is gated by a hysteresis threshold whose
published default is 3.0, twice the first setting (section 3, "Where the
time goes", the step-time table and the paragraph after it); a fingerprint
of every expert is taken at boot and, after swapping, every expert that
moved plus a sample are fingerprinted again wherever they now live, and must
match (section 4, "Does it change the answers?", the table of checks).

The pages give the rule in words only.  Readings taken here:

* Pick counts: each layer counts, per expert, the (token, pick) pairs routed
  to it; ids outside [0, E) are not counted.
* Score: an exponentially decayed pick count, updated once per manager tick
  as score <- decay * score + counts (counts since the previous tick), in
  float64, the product rounded before the sum.
* Swap rule (one layer, one tick): cold experts in decreasing score, hot
  experts in increasing score (equal scores: lower expert index first); the
  i-th cold replaces the i-th hot while
  score_cold > threshold * max(score_hot, min_score), at most max_swaps
  times.  A promoted expert takes the demoted one's HBM slot and the demoted
  one takes the promoted one's cold slot, so both pools keep their sizes.
  The threshold is the hysteresis: a demoted expert needs threshold times
  its replacement's score to come back.
* Fingerprint: the sum modulo 2^64 of SplitMix64's output function (Steele,
  Lea and Flood, "Fast splittable pseudorandom number generators", 2014;
  the finaliser with Stafford's Mix13 constants) applied to
  w_i + (i + 1) * 0x9E3779B97F4A7C15, over the blob's little-endian 64-bit
  words w_i, i = 0, 1, ...  A word of zeros at position 0 therefore
  fingerprints to SplitMix64's first output from seed 0, and position
  enters every term, so moved or reordered bytes change the sum.
"""
import numpy as np

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def count_picks(ids, n_experts):
    """[E] int64: (token, pick) pairs routed to each expert; ids outside [0, E) ignored."""
    a = np.asarray(ids, dtype=np.int64).reshape(-1)
    a = a[(a >= 0) & (a < n_experts)]
    return np.bincount(a, minlength=n_experts)


def mix64(z):
    """SplitMix64's output function on uint64 (numpy arrays wrap modulo 2^64)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def fingerprint(blob):
    """Fingerprint of a byte string whose length is a multiple of 8 (int)."""
    b = np.ascontiguousarray(np.asarray(blob, dtype=np.uint8).reshape(-1))
    if b.size % 8:
        raise ValueError("blob length must be a multiple of 8")
    w = b.view("<u8").astype(np.uint64)
    pos = (np.arange(1, w.size + 1, dtype=np.uint64) * np.uint64(GOLDEN_GAMMA))
    with np.errstate(over="ignore"):
        terms = mix64(w + pos)
    # sum modulo 2^64: numpy's uint64 add wraps
    return int(np.sum(terms, dtype=np.uint64))


def update_scores(score, counts, decay):
    """score <- decay * score + counts (float64; product rounded, then the sum)."""
    prod = np.float64(decay) * np.asarray(score, dtype=np.float64)
    return prod + np.asarray(counts, dtype=np.float64)


def plan_swaps(slot, score, threshold, min_score, max_swaps):
    """Swap pairs [(cold expert, hot expert)] for one layer and the residency
    table after them (a new array)."""
    slot = np.array(slot, dtype=np.int32, copy=True)
    score = np.asarray(score, dtype=np.float64)
    E = slot.size
    cold = sorted((e for e in range(E) if slot[e] < 0), key=lambda e: (-score[e], e))
    hot = sorted((e for e in range(E) if slot[e] >= 0), key=lambda e: (score[e], e))
    pairs = []
    for c, h in zip(cold, hot):
        if len(pairs) >= max_swaps:
            break
        if not score[c] > np.float64(threshold) * max(score[h], np.float64(min_score)):
            break
        pairs.append((c, h))
        slot[c], slot[h] = slot[h], slot[c]
    return pairs, slot


def manager_tick(slot, score, counts, decay, threshold, min_score, max_swaps):
    """One manager tick for one layer: (pairs, new slot, new score)."""
    score = update_scores(score, counts, decay)
    pairs, slot = plan_swaps(slot, score, threshold, min_score, max_swaps)
    return pairs, slot, score


def apply_swaps(slot, pairs, hot_pool, host_pool):
    """Pool contents after the moves (new arrays): the promoted expert's bytes
    into the demoted one's HBM slot, the demoted one's into the promoted one's
    cold slot.  slot is the table BEFORE the swaps."""
    hot_pool = np.array(hot_pool, copy=True)
    host_pool = np.array(host_pool, copy=True)
    for c, h in pairs:
        i, j = int(slot[h]), -int(slot[c]) - 1
        hot_pool[i], host_pool[j] = host_pool[j].copy(), hot_pool[i].copy()
    return hot_pool, host_pool
