"""SwiGLU expert FFN and the weighted top-k combine.

The offloaded planes are the routed experts' w13 (gate and up) and w2 (down)
(GB300 write-up, flag table, --cpu-offload-params row); P3 calls w2 "one of
the large weight planes inside the model's routed expert feed-forward path"
("Five layers made the difference").  Readings taken: the expert is a SwiGLU
FFN, y = W2 (silu(W1 x) * (W3 x)) with silu(g) = g / (1 + e^-g), computed in
fp32 (products of bf16 activations and MXFP4 weights are exact in fp32; the
sums round).  The layer output is sum_j w_j * y_{e_j}, added in the order of
the picks (the gracetier write-up, section 4, notes that the adding order
moves the last decimals, so the order is fixed here) and kept in fp32.
"""
import numpy as np


def silu(g):
    """g * sigmoid(g) = g / (1 + exp(-g)); exp overflow gives -0 for g << 0."""
    with np.errstate(over="ignore"):
        return g / (1 + np.exp(-g))


def expert_ffn(x, w13, w2, dtype=np.float32):
    """One expert on activations x [n][H]: returns y [n][H] in `dtype`.

    w13 [2I][H] (rows 0..I-1 gate, I..2I-1 up), w2 [H][I], both exact."""
    x = np.asarray(x, dtype=dtype)
    w13 = np.asarray(w13, dtype=dtype)
    w2 = np.asarray(w2, dtype=dtype)
    inter = w13.shape[0] // 2
    g = x @ w13[:inter].T          # gate projection [n][I]
    u = x @ w13[inter:].T          # up projection   [n][I]
    h = (silu(g) * u).astype(dtype)
    return h @ w2.T                # down projection [n][H]


def combine(w, y, dtype=np.float32):
    """out[t] = sum_{j=0..k-1} w[t,j] * y[t,j], accumulated in j order.

    w [T][k], y [T][k][H] -> out [T][H]."""
    w = np.asarray(w, dtype=dtype)
    y = np.asarray(y, dtype=dtype)
    out = np.zeros((y.shape[0], y.shape[2]), dtype=dtype)
    for j in range(y.shape[1]):
        out = (out + w[:, j:j + 1] * y[:, j, :]).astype(dtype)
    return out
