"""Direct read of the cold experts (residency scratch == the pinned host pool):
the FFN reads each picked cold expert in place over the host link and nothing
is gathered.  The FFN runs the same tile code on the same bytes, so the output
must be bit-identical to gather-then-compute and to every expert resident,
at decode sizes (one-launch selection path) and past them (grouping + GEMM
path); moe_gather_cold enqueues nothing."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from oracle import gather as ogather  # noqa: E402
from oracle import layer as olayer  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_setup import Layer  # noqa: E402

TOL = 2e-2
TIGHT = 1e-3


def boost_cold(layers, delta):
    """Raise the router bias of the cold experts by delta (same in every layer object)."""
    base = layers[0]
    bias = base.bias_np.copy()
    bias[base.cold] += np.float32(delta)
    for L in layers:
        L.bias_np = bias
        L.bias.copy_(torch.from_numpy(bias))


@pytest.mark.parametrize("T,delta", [(1, 3.0), (8, 0.0), (8, 3.0), (32, 3.0), (40, 3.0)])
def test_direct_read_equals_gather_and_all_resident(T, delta):
    wl = gen.workload("hotcold8")
    g = Layer(wl, T=T)
    d = Layer(wl, T=T, host=g.host, direct=True)   # the same pinned pool, read in place
    hot = Layer(wl, T=T, all_hot=True)
    try:
        if delta:
            boost_cold([g, d, hot], delta)
        a = g.forward().clone()
        b = d.forward().clone()
        c = hot.forward()
        torch.cuda.synchronize()
        ids = d.ids.cpu().numpy()
        pc = ogather.picked_cold(ids, d.slot_np)
        print(f"T={T} delta={delta}: picked cold {len(pc)}", flush=True)
        if delta:
            assert len(pc) >= 1
        assert torch.equal(g.ids, d.ids) and torch.equal(d.ids, hot.ids)
        assert torch.equal(a, b), "direct read changed the output bits"
        assert torch.equal(b, c), "direct read differs from every expert resident"
        # the FFN entry point alone, on the routing just produced
        out = torch.empty_like(b)
        moe.moe_expert_ffn(d.shape, d.x, d.ids, d.w, d.residency, out, d.ws)
        torch.cuda.synchronize()
        assert torch.equal(out, b)
        rows = sorted({0, T // 2, T - 1})
        ref = olayer.layer_forward(d.x_np[rows], d.wr_np, d.bias_np, d.blob, d.H, d.I, d.k)
        assert np.array_equal(ids[rows], ref["ids"])
        err = olayer.max_err_over_rms(b.cpu().numpy()[rows], ref["out"])
        assert err <= TOL and err <= TIGHT, err
    finally:
        g.close()
        d.close()
        hot.close()


def test_direct_read_gather_copies_nothing():
    wl = gen.workload("hotcold8")
    d = Layer(wl, T=8, direct=True)
    try:
        boost_cold([d], 3.0)
        d.forward()
        torch.cuda.synchronize()
        before = d.host.np.copy()
        moe.moe_gather_cold(d.shape, d.ids, d.residency, d.ws)
        torch.cuda.synchronize()
        assert np.array_equal(d.host.np, before)
    finally:
        d.close()
