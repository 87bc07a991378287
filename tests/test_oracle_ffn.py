"""Pins for oracle.ffn and oracle.layer.

Against: a scalar float64 brute force on the tiny shape (its own byte
offsets, the OCP table, exact-rational routing), and closed forms — all-zero
codes give 0; one nonzero per row gives silu(x_a) * x_b placed analytically;
one more on every w2 scale byte doubles the output exactly; identical
experts give a single expert's output; k = 1 gives that expert's output."""
import math

import numpy as np
import pytest

from oracle import blob, ffn, layer, route
from synth import gen
from tests import brute

H, I, E, K, T = 256, 128, 8, 2, 4        # the tiny workload's shape


def _inputs(seed=0):
    x = gen.tokens_bf16(seed, 0, T, H)
    wr = gen.router_weight(seed, 0, E, H)
    blobs = {e: gen.expert_blob(seed, 0, e, H, I) for e in range(E)}
    return x, wr, blobs


@pytest.mark.slow
def test_layer_matches_scalar_bruteforce():
    x, wr, blobs = _inputs()
    res = layer.layer_forward(x, wr, None, lambda e: blobs[e], H, I, K)
    ref = np.zeros((T, H))
    for t in range(T):
        z = brute.exact_logits(x[t], wr)
        ids = brute.topk_bruteforce(z, K)
        assert res["ids"][t].tolist() == ids
        w = brute.softmax_weights(z, ids)
        xt = [float(v) for v in route.bf16_bits_to_f32(x[t])]
        acc = [0.0] * H
        for j, e in enumerate(ids):
            y = brute.expert_ffn_scalar(xt, blobs[e], H, I)
            acc = [acc[r] + w[j] * y[r] for r in range(H)]
        ref[t] = acc
    err = layer.max_err_over_rms(res["out"], ref)
    assert err < 1e-5, err


def _zero_blob():
    return np.zeros(gen.expert_bytes(H, I), dtype=np.uint8)


def _set_scales(b, value_fn):
    """b with every scale byte (row, block) set to value_fn((row, block))."""
    w13q, w13s, w2q, w2s = blob.split(b, H, I)
    for arr in (w13s, w2s):
        for idx in np.ndindex(arr.shape):
            arr[idx] = value_fn(idx)
    return blob.join(w13q, w13s, w2q, w2s)


def _put(codes_view, r, c, code):
    byte = int(codes_view[r, c // 2])
    if c % 2:
        byte = (byte & 0x0F) | (code << 4)
    else:
        byte = (byte & 0xF0) | code
    codes_view[r, c // 2] = byte


def test_all_zero_codes_give_zero():
    rng = np.random.default_rng(0)
    b = _set_scales(_zero_blob(), lambda idx: int(rng.integers(100, 140)))
    w13, w2 = blob.weights(b, H, I)
    x = route.bf16_bits_to_f32(gen.tokens_bf16(0, 0, T, H))
    y = ffn.expert_ffn(x, w13, w2)
    assert np.all(y == 0)


def test_one_nonzero_per_row_closed_form():
    rng = np.random.default_rng(1)
    b = _set_scales(_zero_blob(), lambda idx: 127)
    w13q, w13s, w2q, w2s = blob.split(b, H, I)
    a = rng.integers(0, H, I)           # gate row j reads x[a_j]
    bb = rng.integers(0, H, I)          # up row j reads x[b_j]
    c = rng.integers(0, I, H)           # down row r reads h[c_r]
    sg = rng.integers(124, 130, I)
    su = rng.integers(124, 130, I)
    s2 = rng.integers(124, 130, H)
    for j in range(I):
        _put(w13q, j, a[j], 2)           # code 2 = 1.0
        _put(w13q, I + j, bb[j], 2)
        w13s[j, a[j] // 32] = sg[j]
        w13s[I + j, bb[j] // 32] = su[j]
    for r in range(H):
        _put(w2q, r, c[r], 2)
        w2s[r, c[r] // 32] = s2[r]
    b = blob.join(w13q, w13s, w2q, w2s)
    w13, w2 = blob.weights(b, H, I)
    xb = gen.tokens_bf16(3, 0, T, H)
    x = route.bf16_bits_to_f32(xb).astype(np.float64)
    y = ffn.expert_ffn(x, w13, w2)
    for t in range(T):
        h = []
        for j in range(I):
            g = math.ldexp(x[t, a[j]], int(sg[j]) - 127)
            u = math.ldexp(x[t, bb[j]], int(su[j]) - 127)
            h.append(g / (1 + math.exp(-g)) * u)
        want = np.array([math.ldexp(h[c[r]], int(s2[r]) - 127) for r in range(H)])
        np.testing.assert_allclose(y[t], want, rtol=2e-6, atol=0)


def test_w2_scale_plus_one_doubles_exactly():
    x, wr, blobs = _inputs(1)
    b0 = blobs[3]
    w13q, w13s, w2q, w2s = blob.split(b0, H, I)
    b1 = blob.join(w13q, w13s, w2q, w2s + 1)
    xf = route.bf16_bits_to_f32(x)
    y0 = ffn.expert_ffn(xf, *blob.weights(b0, H, I))
    y1 = ffn.expert_ffn(xf, *blob.weights(b1, H, I))
    assert np.array_equal(y1, 2 * y0)


def test_identical_experts_equal_single_expert():
    x, wr, blobs = _inputs(2)
    res = layer.layer_forward(x, wr, None, lambda e: blobs[5], H, I, K)
    single = ffn.expert_ffn(route.bf16_bits_to_f32(x), *blob.weights(blobs[5], H, I))
    assert layer.max_err_over_rms(res["out"], single) < 1e-6


def test_k1_is_the_single_picked_expert():
    x, wr, blobs = _inputs(3)
    res = layer.layer_forward(x, wr, None, lambda e: blobs[e], H, I, 1)
    assert np.all(res["w"] == 1.0)
    xf = route.bf16_bits_to_f32(x)
    for t in range(T):
        e = int(res["ids"][t, 0])
        y = ffn.expert_ffn(xf[t:t + 1], *blob.weights(blobs[e], H, I))
        # w = 1 exactly; BLAS may round a 1-row product differently from the
        # batched one, so compare to fp32 rounding
        assert layer.max_err_over_rms(res["out"][t], y[0]) < 1e-6


def test_combine_order_and_linearity():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((3, 4, 16)).astype(np.float32)
    w = rng.random((3, 4)).astype(np.float32)
    out = ffn.combine(w, y)
    # j-order accumulation, written out term by term
    want = np.zeros((3, 16), dtype=np.float32)
    for j in range(4):
        want = want + w[:, j:j + 1] * y[:, j]
    assert np.array_equal(out, want)
    w2 = w.copy()
    w2[:, 1] *= 2
    diff = ffn.combine(w2, y).astype(np.float64) - out
    np.testing.assert_allclose(diff, w[:, 1:2] * y[:, 1].astype(np.float64), rtol=1e-5, atol=1e-5)


def test_silu_large_negative_is_signed_zero():
    h = ffn.silu(np.array([-1e4, 0.0, 1e4], dtype=np.float32))
    assert h[0] == 0 and math.copysign(1, h[0]) == -1
    assert h[1] == 0 and h[2] == 1e4


def test_layer_experts_on_threads_give_the_same_bits():
    """The thread-pool evaluation used by the full-size GPU tests changes only
    the order in which independent experts are evaluated."""
    from tests import oracle_threads
    x, wr, blobs = _inputs(3)
    a = layer.layer_forward(x, wr, None, lambda e: blobs[e], H, I, K)
    b = oracle_threads.layer_forward(x, wr, None, lambda e: blobs[e], H, I, K)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["out"], b["out"])
