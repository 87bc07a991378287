"""Calibrate the correlation of the synthetic speculative-verify windows
(offline script; test infrastructure like the rest of oracle/).

Writes synth/verify_calibration.json, the input-recipe data that the
generator reads; it routes with the oracle only.  Run once:

    python -m oracle.calibrate_verify [--windows 1024]

Target (the GB300 inference write-up, the table of what was tried, the
speculative-fetching row): a verify window of 1 + 5 tokens touches 3.7x the
distinct experts of one token.  One token touches top_k = 6 experts, so a
window touches 22.2 distinct experts on average.

Readings taken: the tokens of a window are synth.gen.verify_tokens_bf16
(a shared component with correlation rho, bf16-rounded); routing is the
layer's router plus its Zipf prior (synth.gen.zipf_prior at the calibrated
alpha), top-6 as the oracle selects; rho is one number, set by bisection on
layer 0; the other layers are reported, not fitted.
"""
import argparse
import json

import numpy as np

from oracle.route import router_logits, select_topk
from synth import gen

E, H, K = 384, 4096, 6
SEED, CAL_SEED = 0, 2
TARGET = 3.7
WINDOW = 6


def unique_per_window(seed, layer, windows, window, rho, alpha):
    x = gen.verify_tokens_bf16(seed, layer, windows, window, H, rho)
    z = router_logits(x, gen.router_weight(SEED, layer, E, H), gen.zipf_prior(SEED, layer, E, alpha))
    ids = select_topk(z, K).reshape(windows, window * K)
    return np.array([len(np.unique(r)) for r in ids], dtype=np.float64)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--windows", type=int, default=1024)
    ap.add_argument("--report-layers", type=int, default=8)
    ap.add_argument("--out", default=gen.VERIFY_CALIBRATION_PATH)
    a = ap.parse_args()
    alpha = gen.load_calibration()["alpha"]

    lo, hi = 0.0, 1.0
    for _ in range(20):
        mid = 0.5 * (lo + hi)
        m = unique_per_window(CAL_SEED, 0, a.windows, WINDOW, mid, alpha).mean() / K
        print(f"rho {mid:.6f}: {m:.4f}x", flush=True)
        if m > TARGET:
            lo = mid
        else:
            hi = mid
    rho = round(0.5 * (lo + hi), 6)

    stats = {}
    for layer in range(a.report_layers):
        u6 = unique_per_window(CAL_SEED, layer, a.windows, 6, rho, alpha)
        u2 = unique_per_window(CAL_SEED, layer, a.windows, 2, rho, alpha)
        stats[str(layer)] = {"window6_x": round(float(u6.mean() / K), 4),
                             "window2_x": round(float(u2.mean() / K), 4)}
        print(f"layer {layer}: window 6 {u6.mean() / K:.3f}x, window 2 {u2.mean() / K:.3f}x", flush=True)

    with open(a.out, "w") as f:
        json.dump({"rho": rho, "target_multiplier": TARGET, "window": WINDOW, "top_k": K,
                   "alpha": alpha, "calib_seed": CAL_SEED, "calib_windows": a.windows,
                   "stats": stats}, f, indent=1)
    print("wrote", a.out)


if __name__ == "__main__":
    main()
