"""Router: logits, top-k selection and routing weights.

The pages: per token a small router chooses 6 of the 384 experts (the
inference-engineering write-up, "Milo and James try inference engineering",
first paragraph on the mixture-of-experts design).  They give no score function; the readings taken:

  * scores are a softmax over the E logits z[t,e] = sum_h x[t,h] Wr[e,h] + b[e],
    b an optional logit prior (the synthetic Zipf bias), added before softmax;
  * the k largest are kept; equal logits go to the lower expert index;
  * selection is made on the logits (softmax is strictly increasing, so the
    set is the same, without ties made by exp rounding);
  * the kept weights are renormalised to sum to 1 (renormalize=True), or are
    the plain softmax probabilities (renormalize=False);
  * the k picks are listed by decreasing weight, ties by increasing index;
  * no shared expert, no group-limited routing, routed scale 1.
"""
import numpy as np


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exactly."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def router_logits(x_bits, w_router, bias=None):
    """z[t,e] = sum_h x[t,h] * Wr[e,h] + b[e] in float64 ([T][E]).

    bf16 x times fp32 Wr is exact in float64, so only the float64 summation
    rounds (relative error ~1e-16)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    wr = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    z = x @ wr.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return z


def select_topk(z, k):
    """ids [T][k]: the k largest z per row, decreasing, ties to the lower index.

    A stable sort of -z keeps equal values in increasing index order."""
    z = np.asarray(z, dtype=np.float64)
    order = np.argsort(-z, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(z, ids, renormalize=True):
    """Softmax weights of the picked experts, float64 [T][k].

    p_e = exp(z_e - max z); renormalize: w_j = p_{ids_j} / sum_j' p_{ids_j'};
    otherwise w_j = p_{ids_j} / sum_e p_e."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    picked = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        return picked / picked.sum(axis=1, keepdims=True)
    return picked / p.sum(axis=1, keepdims=True)


def route(x_bits, w_router, bias, k, renormalize=True):
    """(ids int32 [T][k], weights float64 [T][k], logits float64 [T][E])."""
    z = router_logits(x_bits, w_router, bias)
    ids = select_topk(z, k)
    return ids, topk_weights(z, ids, renormalize), z


def topk_margin(z, k):
    """Gap between the k-th and (k+1)-th largest logit of each row ([T])."""
    z = np.sort(np.asarray(z, dtype=np.float64), axis=1)[:, ::-1]
    if k >= z.shape[1]:
        return np.full(z.shape[0], np.inf)
    return z[:, k - 1] - z[:, k]
