"""One routed-expert layer end to end (route, FFN of every picked expert,
weighted combine).  Where an expert lives (HBM or host) does not enter: the
gracetier write-up (section 1) runs every picked expert in one call as though
all of them were resident in HBM, so the oracle reads each expert's bytes
from wherever the caller keeps them."""
import numpy as np

from . import blob as _blob
from .ffn import combine, expert_ffn
from .route import bf16_bits_to_f32, route


def layer_forward(x_bits, w_router, bias, blob_of, H, I, k, renormalize=True,
                  dtype=np.float32, map_fn=map):
    """x_bits [T][H] bf16 bits, w_router [E][H] fp32, bias [E] fp32 or None,
    blob_of(e) -> uint8 blob of expert e.

    The picked experts are independent: map_fn(f, experts) evaluates f on
    each (the builtin map by default; a thread pool's map gives the same
    numbers, each expert's arithmetic being the same).

    Returns dict(ids [T][k] int32, w [T][k] float64, z [T][E] float64,
    y [T][k][H], out [T][H] in `dtype`)."""
    ids, w, z = route(x_bits, w_router, bias, k, renormalize)
    x = bf16_bits_to_f32(x_bits)
    T = x.shape[0]
    y = np.zeros((T, k, H), dtype=dtype)

    def one_expert(e):
        w13, w2 = _blob.weights(blob_of(int(e)), H, I)
        tt, jj = np.nonzero(ids == e)
        return tt, jj, expert_ffn(x[tt], w13, w2, dtype)

    for tt, jj, ye in map_fn(one_expert, np.unique(ids)):
        y[tt, jj] = ye
    out = combine(w.astype(dtype), y, dtype)
    return {"ids": ids, "w": w, "z": z, "y": y, "out": out}


def rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a)))


def max_err_over_rms(got, ref):
    """max |got - ref| / RMS(ref): the layer-output parity measure."""
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)) / rms(ref))
