"""Exact ties in the router logits, on every top-k path of the HIP library.

Expert indices must be bit-exact with the oracle, and equal logits go to the
lower expert index.  Random logits almost never tie, so the router is built to
make them tie exactly: experts of one group share one router row and one bias
value, so their fp32 logits are the same bits whatever order the sums take
(and the oracle's fp64 logits are equal too).  The groups' biases put them far
above every other expert:

  group A {5, 69}        bias +100  picks 0, 1  (same lane, different slots)
  group B {131, 70, 3}   bias  +90  picks 2..4  (three lanes and slots)
  group C {383, 200}     bias  +80  pick 5: 200 only; 383 is the first expert
                                     left out, so the tie sits at the k-th place

Paths (H=256, I=128, E=384, k=6 keeps every expert small):
  moe_route T<=32 (route_logits_small + route_topk) and T>32 (router GEMM
  with 64- and 128-token tiles + route_topk); moe_layer_forward at T=1 (every
  gate/up block selects for itself), T=2..5 (select_group_small), T=8 with
  group C cold (the gather's own top-k, gather_cold_sel, beside the grouping)
  and T=40 (route_topk + chunked grouping).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from oracle import gather as ogather  # noqa: E402
from oracle import layer as olayer  # noqa: E402
from oracle import route as oroute  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_setup import Layer  # noqa: E402

GROUPS = ((100.0, (5, 69)), (90.0, (131, 70, 3)), (80.0, (383, 200)))
WANT = [5, 69, 3, 70, 131, 200]


def tie_workload(T, n_hot=None):
    return gen.Workload("ties", 256, 128, 384, 6, T, n_hot=n_hot, seed=11)


def make_ties(L):
    """Give each group one router row and one bias value (oracle and GPU)."""
    wr = L.wr_np.copy()
    bias = np.zeros(L.E, dtype=np.float32) if L.bias_np is None else L.bias_np.copy()
    for b, members in GROUPS:
        for e in members:
            wr[e] = wr[members[0]]
            bias[e] = np.float32(b)
    L.wr_np, L.bias_np = wr, bias
    L.wr.copy_(torch.from_numpy(wr))
    L.bias = torch.from_numpy(bias).cuda()


def route(L, renorm=True):
    z = torch.empty((L.T, L.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((L.T, L.k), dtype=torch.int32, device="cuda")
    w = torch.empty((L.T, L.k), dtype=torch.float32, device="cuda")
    moe.moe_route(L.shape, L.x, L.wr, L.bias, renorm, ids, w, z, L.ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), z.cpu().numpy()


def check_tied_logits(z):
    """The GPU logits of each group are the same bits (the test's premise)."""
    zb = z.view(np.uint32)
    for _, members in GROUPS:
        for e in members[1:]:
            assert np.array_equal(zb[:, e], zb[:, members[0]]), (members, e)


@pytest.mark.parametrize("T", [1, 7, 32, 33, 4100])
def test_route_ties_lower_index(T):
    L = Layer(tie_workload(T))
    make_ties(L)
    ids, w, z = route(L)
    check_tied_logits(z)
    assert np.all(ids == np.array(WANT, dtype=np.int32)[None, :]), ids[:4]
    ref = oroute.route(L.x_np, L.wr_np, L.bias_np, L.k)
    assert np.array_equal(ids, ref[0])
    # R1: the oracle's selection on the GPU's own logits
    assert np.array_equal(oroute.select_topk(z.astype(np.float64), L.k), ids)
    # tied picks get the same weight bits
    assert np.array_equal(w[:, 0], w[:, 1])
    assert np.array_equal(w[:, 2], w[:, 3]) and np.array_equal(w[:, 3], w[:, 4])
    assert np.max(np.abs(w - ref[1])) <= 2e-6


@pytest.mark.parametrize("T", [1, 2, 5, 32, 40])
def test_layer_ties_all_resident(T):
    """T=1: selection inside every gate/up block; T=2, 5: select_group_small;
    T=32: its block-wide grouping; T=40: route_topk and the chunked grouping."""
    L = Layer(tie_workload(T))
    make_ties(L)
    out = L.forward()
    torch.cuda.synchronize()
    ids = L.ids.cpu().numpy()
    assert np.all(ids == np.array(WANT, dtype=np.int32)[None, :])
    rows = sorted({0, T - 1})
    ref = olayer.layer_forward(L.x_np[rows], L.wr_np, L.bias_np, L.blob, L.H, L.I, L.k)
    assert np.array_equal(ids[rows], ref["ids"])
    assert olayer.max_err_over_rms(out.cpu().numpy()[rows], ref["out"]) <= 1e-3


@pytest.mark.parametrize("T", [1, 3, 8, 32])
def test_layer_ties_cold_group_gathers_lower_index(T):
    """Group C's two experts are cold: only expert 200's slot is gathered
    (T=1: the hot gate/up blocks publish the pick set; T=3: select_group_small
    then the gather; T=8, 32: the gather's own top-k on the side stream)."""
    wl = tie_workload(T, n_hot=382)
    hot = [e for e in range(384) if e not in (200, 383)]
    L = Layer(wl, hot=hot)
    try:
        make_ties(L)
        L.scratch.fill_(0xEE)
        out = L.forward()
        torch.cuda.synchronize()
        ids = L.ids.cpu().numpy()
        assert np.all(ids == np.array(WANT, dtype=np.int32)[None, :])
        pc = ogather.picked_cold(ids, L.slot_np)
        assert pc.tolist() == [200]
        s200, s383 = -int(L.slot_np[200]) - 1, -int(L.slot_np[383]) - 1
        scratch = L.scratch.cpu().numpy()
        host = L.host.np.reshape(L.n_cold, L.B)
        assert np.array_equal(scratch[s200], host[s200])
        assert np.all(scratch[s383] == 0xEE), "the tied expert with the higher index was gathered"
        rows = sorted({0, T - 1})
        ref = olayer.layer_forward(L.x_np[rows], L.wr_np, L.bias_np, L.blob, L.H, L.I, L.k)
        assert olayer.max_err_over_rms(out.cpu().numpy()[rows], ref["out"]) <= 1e-3
    finally:
        L.close()


@pytest.mark.parametrize("T", [1, 40])
def test_nan_router_row_ranks_last(T):
    """A NaN logit ranks after -inf (the oracle's order): expert 0's router row
    is NaN and every other expert but five has bias -inf, so the sixth pick is
    expert 1 (logit -inf), not expert 0 (NaN)."""
    L = Layer(tie_workload(T))
    wr = L.wr_np.copy()
    wr[0] = np.nan
    bias = np.full(L.E, -np.inf, dtype=np.float32)
    top = [7, 50, 100, 250, 300]
    bias[top] = np.float32(10.0)
    L.wr_np, L.bias_np = wr, bias
    L.wr.copy_(torch.from_numpy(wr))
    L.bias = torch.from_numpy(bias).cuda()
    ids, w, z = route(L)
    assert np.all(np.isnan(z[:, 0])) and np.all(z[:, 1] == -np.inf)
    ref_ids = oroute.select_topk(oroute.router_logits(L.x_np, wr, bias), L.k)
    assert np.array_equal(ids, ref_ids)
    assert np.all(ids[:, 5] == 1)
    assert np.all(w[:, 5] == 0.0)
