"""Input recipes: the drifted Zipf prior, and the speculative-verify
recipe: the draft schedule, the window
correlation of the generated tokens, and the distinct-expert multiplier the
calibration fitted (3.7x one token's experts for a 1 + 5 window, the GB300
inference write-up, speculative-fetching row of its table of what was
tried), re-measured on tokens the calibration never saw."""
import numpy as np
import pytest

from oracle.route import bf16_bits_to_f32, router_logits, select_topk
from synth import gen


def test_draft_schedule():
    assert [gen.verify_window(s) for s in (1, 2, 3, 4)] == [6] * 4
    assert [gen.verify_window(s) for s in (5, 8, 16)] == [2] * 3
    for bad in (0, 17):
        with pytest.raises(ValueError):
            gen.verify_window(bad)


def test_window_correlation():
    rho = 0.3
    x = bf16_bits_to_f32(gen.verify_tokens_bf16(5, 0, 64, 6, 1024, rho)).reshape(64, 6, 1024)
    x = x.astype(np.float64)
    assert abs(x.var() - 1.0) < 0.02
    within = np.mean([np.corrcoef(x[s, 0], x[s, j])[0, 1] for s in range(64) for j in range(1, 6)])
    across = np.mean([np.corrcoef(x[s, 0], x[s + 1, 0])[0, 1] for s in range(63)])
    assert abs(within - rho) < 0.02
    assert abs(across) < 0.02
    # rho = 0: the windows' tokens are independent; rho = 1: all equal
    y = gen.verify_tokens_bf16(5, 0, 2, 3, 64, 1.0).reshape(2, 3, 64)
    assert np.array_equal(y[:, 0], y[:, 1]) and not np.array_equal(y[0, 0], y[1, 0])


@pytest.mark.slow
def test_calibrated_multiplier_on_fresh_tokens():
    cal = gen.load_verify_calibration()
    zipf = gen.load_calibration()
    assert cal["alpha"] == zipf["alpha"]
    E, H, K, W, n = 384, 4096, 6, cal["window"], 256
    for layer in (1, 5):
        x = gen.verify_tokens_bf16(11, layer, n, W, H, cal["rho"])
        z = router_logits(x, gen.router_weight(0, layer, E, H), gen.zipf_prior(0, layer, E, zipf["alpha"]))
        ids = select_topk(z, K).reshape(n, W * K)
        mult = np.mean([len(np.unique(r)) for r in ids]) / K
        assert abs(mult - cal["target_multiplier"]) < 0.15, (layer, mult)
        # without the shared component the window would touch far more experts
        x0 = gen.verify_tokens_bf16(11, layer, n, W, H, 0.0)
        z0 = router_logits(x0, gen.router_weight(0, layer, E, H), gen.zipf_prior(0, layer, E, zipf["alpha"]))
        ids0 = select_topk(z0, K).reshape(n, W * K)
        assert np.mean([len(np.unique(r)) for r in ids0]) / K > mult + 0.3


def test_drifted_prior():
    """Drift keeps the prior's values (a permutation of the same ranks) and
    moves about frac of them per round; zero rounds is the calibrated prior."""
    alpha = gen.load_calibration()["alpha"]
    base = gen.zipf_prior(0, 3, 384, alpha)
    assert np.array_equal(gen.drifted_zipf_prior(0, 3, 384, alpha, 0.3, 0), base)
    d1 = gen.drifted_zipf_prior(0, 3, 384, alpha, 0.3, 1)
    d2 = gen.drifted_zipf_prior(0, 3, 384, alpha, 0.3, 2)
    assert np.array_equal(np.sort(d1), np.sort(base)) and np.array_equal(np.sort(d2), np.sort(base))
    moved1 = int(np.sum(d1 != base))
    assert 0.2 * 384 < moved1 <= 0.3 * 384 + 1
    assert np.sum(d2 != base) > moved1
    assert np.array_equal(gen.drifted_zipf_prior(0, 3, 384, alpha, 0.3, 1), d1)
