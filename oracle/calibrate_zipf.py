"""Calibrate the synthetic Zipf routing prior and the hot sets (offline script).

Writes synth/zipf_calibration.json, the input-recipe data that the generator
reads; it routes with the oracle only.  Run once:

    python -m oracle.calibrate_zipf [--layers 40] [--tokens 65536]

Targets (the pages' routing statistics):
  * 98.7% of expert lookups hit 73% of the experts — the GB300 inference
    write-up, paragraph on hot/cold doors closed by the hardware;
  * 255 hot experts per layer, 129 cold — the gracetier write-up, section 1.

Readings taken: the prior is b_e = -alpha * 1.1 * ln(rank_e) with a seeded
rank permutation per layer (synth.gen.zipf_prior); alpha is one number, set
by bisection on layer 0 so that the 280 most-picked experts (73% of 384)
receive 98.7% of the top-6 picks of the calibration tokens; the hot set of a
layer is its 255 most-picked experts in that sample (ties to the lower
index).  The calibration tokens (seed 1) are shared by every layer.
"""
import argparse
import json
import time

import numpy as np

from oracle.route import router_logits, select_topk
from synth import gen

E, H, K = 384, 4096, 6
SEED, CAL_SEED = 0, 1
TARGET_EXPERTS, TARGET_FRAC = 280, 0.987
N_HOT = 255


def _counts(z, bias, alpha):
    ids = select_topk(z + alpha * bias[None, :].astype(np.float64), K)
    return np.bincount(ids.reshape(-1), minlength=E)


def _top_share(counts, n):
    order = np.argsort(-counts, kind="stable")
    return counts[order[:n]].sum() / counts.sum(), order[:n]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--tokens", type=int, default=65536)
    ap.add_argument("--out", default=gen.CALIBRATION_PATH)
    a = ap.parse_args()

    x = gen.tokens_bf16(CAL_SEED, 0, a.tokens, H)
    unit = {}

    def logits(layer):
        if layer not in unit:
            unit[layer] = router_logits(x, gen.router_weight(SEED, layer, E, H), None)
        return unit[layer]

    # b(alpha) = alpha * b(1): calibrate alpha on layer 0 by bisection
    b1 = gen.zipf_prior(SEED, 0, E, 1.0).astype(np.float64)
    z0 = logits(0)
    lo, hi = 0.0, 2.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        share, _ = _top_share(_counts(z0, b1, mid), TARGET_EXPERTS)
        if share < TARGET_FRAC:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi), 6)
    print(f"alpha = {alpha}", flush=True)

    hot, stats = {}, {}
    for layer in range(a.layers):
        t0 = time.time()
        bias = gen.zipf_prior(SEED, layer, E, alpha).astype(np.float64)
        z = logits(layer) if layer == 0 else router_logits(x, gen.router_weight(SEED, layer, E, H), None)
        ids = select_topk(z + bias[None, :], K)
        c = np.bincount(ids.reshape(-1), minlength=E)
        s280, _ = _top_share(c, TARGET_EXPERTS)
        s255, h = _top_share(c, N_HOT)
        hot[f"{SEED}:{layer}"] = sorted(int(e) for e in h)
        stats[f"{SEED}:{layer}"] = {"share_top280": round(float(s280), 5),
                                   "share_hot255": round(float(s255), 5)}
        unit.pop(layer, None)
        print(f"layer {layer}: top280 {s280:.4f} hot255 {s255:.4f} ({time.time() - t0:.1f}s)", flush=True)

    with open(a.out, "w") as f:
        json.dump({"alpha": alpha, "s": 1.1, "calib_seed": CAL_SEED, "calib_tokens": a.tokens,
                   "target": {"experts": TARGET_EXPERTS, "share": TARGET_FRAC}, "n_hot": N_HOT,
                   "stats": stats, "hot": hot}, f, indent=0)
    print("wrote", a.out)


if __name__ == "__main__":
    main()
