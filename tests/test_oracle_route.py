"""Pins for oracle.route: logits, top-k and weights.

Against: exact rational logits and a search over every k-subset (tiny E),
forced ties, the k=2 closed form (w0 = sigmoid(z0 - z1)), shift invariance,
scipy's softmax for the unnormalised case, and the bf16 bit-pattern table."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle import route
from synth import gen
from tests import brute


def _tiny(E, H, T, seed):
    x = gen.tokens_bf16(seed, 0, T, H)
    wr = gen.router_weight(seed, 0, E, H)
    return x, wr


def test_bf16_bits_table():
    with open(os.path.join(brute.GOLDEN, "bf16_bits.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for hx, val in rows:
        got = float(route.bf16_bits_to_f32(np.array([int(hx, 16)], dtype=np.uint16))[0])
        want = math.ldexp(1.0, int(val[2:])) if val.startswith("2^") else float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), hx


@pytest.mark.parametrize("E,k,H,T,seed", [(8, 2, 32, 4, 0), (16, 4, 16, 3, 1), (8, 3, 24, 3, 2)])
def test_topk_and_weights_bruteforce(E, k, H, T, seed):
    x, wr = _tiny(E, H, T, seed)
    bias = gen.zipf_prior(seed, 0, E, 0.7)
    ids, w, z = route.route(x, wr, bias, k)
    for t in range(T):
        zt = brute.exact_logits(x[t], wr, bias)
        # float64 logits are the exact ones rounded once per term: tiny error
        assert max(abs(float(zt[e]) - z[t, e]) for e in range(E)) < 1e-12
        want = brute.topk_bruteforce(zt, k)
        assert ids[t].tolist() == want
        ww = brute.softmax_weights(zt, want)
        assert np.allclose(w[t], ww, rtol=0, atol=1e-12)


def test_forced_ties_pick_lower_index():
    E, H, k = 8, 16, 3
    x, wr = _tiny(E, H, 2, 3)
    wr = wr.copy()
    best = int(np.argmax(route.router_logits(x, wr)[0]))
    # copy the best row into two other experts: a three-way tie at the top
    a, b = [e for e in (1, 6, 2) if e != best][:2]
    wr[a] = wr[best]
    wr[b] = wr[best]
    ids, w, z = route.route(x, wr, None, k)
    tied = sorted({a, b, best})
    assert ids[0].tolist() == tied
    assert np.allclose(w[0], 1.0 / 3, atol=1e-15)


def test_all_equal_logits_give_first_k():
    E, H, k = 8, 16, 4
    x = np.zeros((1, H), dtype=np.uint16)          # all-zero tokens: every logit 0
    _, wr = _tiny(E, H, 1, 0)
    ids, w, _ = route.route(x, wr, None, k)
    assert ids[0].tolist() == [0, 1, 2, 3]
    assert np.all(w[0] == 0.25)


def test_k2_closed_form():
    E, H = 8, 32
    x, wr = _tiny(E, H, 5, 4)
    ids, w, z = route.route(x, wr, None, 2)
    for t in range(5):
        z0, z1 = z[t, ids[t, 0]], z[t, ids[t, 1]]
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(z1 - z0))) < 1e-15
        assert z0 >= z1


def test_shift_invariance_and_sum_to_one():
    E, H, k = 16, 32, 4
    x, wr = _tiny(E, H, 6, 5)
    ids0, w0, _ = route.route(x, wr, None, k)
    ids1, w1, _ = route.route(x, wr, np.full(E, 3.5, dtype=np.float32), k)
    assert np.array_equal(ids0, ids1)
    assert np.allclose(w0, w1, atol=1e-14)
    assert np.allclose(w0.sum(axis=1), 1.0, atol=1e-14)


def test_unnormalised_weights_are_softmax_probabilities():
    E, H, k = 16, 32, 4
    x, wr = _tiny(E, H, 4, 6)
    ids, w, z = route.route(x, wr, None, k, renormalize=False)
    p = softmax(z, axis=1)
    assert np.allclose(w, np.take_along_axis(p, ids.astype(np.int64), axis=1), atol=1e-15)


def test_selection_on_fp32_logits_is_exact():
    # ids from fp32 logits agree with a brute-force sort of the same fp32 values
    rng = np.random.default_rng(0)
    z = rng.standard_normal((50, 12)).astype(np.float32)
    z[:, 3] = z[:, 7]                     # ties
    ids = route.select_topk(z, 5)
    for t in range(50):
        want = brute.topk_bruteforce([Fraction(float(v)) for v in z[t]], 5)
        assert ids[t].tolist() == want


def test_margin():
    z = np.array([[3.0, 1.0, 2.0, 0.5]])
    assert route.topk_margin(z, 2)[0] == 1.0


def test_signed_zeros_tie_to_lower_index():
    """+0 and -0 compare equal, so they tie like any equal logits."""
    z = np.array([[-1.0, -0.0, 0.0, -2.0],
                  [-1.0, 0.0, -0.0, -2.0]])
    assert route.select_topk(z, 1).tolist() == [[1], [1]]
    assert route.select_topk(z, 2).tolist() == [[1, 2], [1, 2]]


def test_nan_logits_rank_after_minus_infinity():
    """Reading taken: a NaN logit ranks below every number (-inf included),
    NaNs among themselves by increasing index."""
    nan, inf = float("nan"), float("inf")
    z = np.array([[nan, -inf, 1.0, nan, -inf, 0.5]])
    assert route.select_topk(z, 6).tolist() == [[2, 5, 1, 4, 0, 3]]
    assert route.select_topk(z, 3).tolist() == [[2, 5, 1]]
