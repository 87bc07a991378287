"""Thread-pool evaluation of the oracle's per-expert loop for full-size
parity checks (test infrastructure).  numpy releases the GIL in the dequant
and the products, so the experts of a layer run in parallel; BLAS is held to
one thread per worker.  The numbers are the oracle's own: only the order in
which independent experts are evaluated changes."""
import concurrent.futures as cf
import os

from threadpoolctl import threadpool_limits

from oracle import layer as olayer


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(n, 16))


def layer_forward(x_bits, w_router, bias, blob_of, H, I, k, renormalize=True):
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(workers()) as ex:
        return olayer.layer_forward(x_bits, w_router, bias, blob_of, H, I, k, renormalize, map_fn=ex.map)
