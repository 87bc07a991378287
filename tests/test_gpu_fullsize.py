"""Full-size parity and the layer's invariants on the GPU.

  * the prefill layer (8192 tokens, 384 experts) on every one of its
    8192 x 4096 outputs against the oracle;
  * one batch-32 layer at the decode shape with 255 hot / 129 cold experts,
    every row;
  * a layer with no resident expert at all (n_hot = 0): every picked expert
    is gathered and the FFN runs on the gathered bytes;
  * relabelling the experts permutes the ids and leaves the output bits;
  * identical experts give one expert's FFN whatever the routing;
  * a layer of a stack never reads a scratch slot it did not gather (the
    scratch poisoned before every layer leaves every output's bits).

The bars and the index rules are those of tests/gpu_checks.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from oracle import blob as oblob  # noqa: E402
from oracle import ffn as offn  # noqa: E402
from oracle import gather as ogather  # noqa: E402
from oracle import route as oroute  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_checks import TIGHT, check_out, check_route, oracle_out, route_on_gpu  # noqa: E402
from tests.gpu_setup import HostBuffer, Layer, fill_host_experts  # noqa: E402


@pytest.mark.timeout(600)
def test_prefill8k_full_parity():
    """Every output of the 8192-token layer.  A token whose oracle margin is
    below twice the logit error may pick differently (R3); its row is then
    left out of the output comparison (counted, and at most a few)."""
    L = Layer(gen.workload("prefill8k"))
    ids_g, w_g, z_g = route_on_gpu(L)
    ties = check_route(L, ids_g, w_g, z_g)
    out = L.forward()
    torch.cuda.synchronize()
    assert np.array_equal(L.ids.cpu().numpy(), ids_g)
    got = out.cpu().numpy()
    ref = oracle_out(L)
    same = np.all(ref["ids"] == ids_g, axis=1)
    print(f"prefill8k: near-tie tokens {ties}, tokens picking differently {int((~same).sum())}", flush=True)
    assert (~same).sum() <= ties
    err = check_out(got[same], ref["out"][same])
    print(f"prefill8k: all {int(same.sum())} x {L.H} outputs, max err / RMS = {err:.2e}")


@pytest.mark.timeout(300)
def test_batch32_hotcold_layer_every_row():
    wl = gen.workload("hotcold8")
    L = Layer(wl, T=32)
    try:
        L.scratch.fill_(0xEE)
        ids_g, w_g, z_g = route_on_gpu(L)
        check_route(L, ids_g, w_g, z_g)
        out = L.forward()
        torch.cuda.synchronize()
        ids = L.ids.cpu().numpy()
        assert np.array_equal(ids, ids_g)
        ref = oracle_out(L)
        assert np.array_equal(ids, ref["ids"])
        err = check_out(out.cpu().numpy(), ref["out"])
        pc = ogather.picked_cold(ids, L.slot_np)
        print(f"batch32 hot/cold: {len(np.unique(ids))} experts, {len(pc)} cold, max err / RMS = {err:.2e}")
    finally:
        L.close()


@pytest.mark.timeout(600)
def test_no_resident_expert():
    """n_hot = 0: the whole layer sits in pinned host memory.  At 1, 8 and 40
    tokens every picked expert is gathered into its slot (and no other slot is
    written), the FFN runs on those bytes, the outputs are the oracle's, and
    at 8 tokens they are bit-identical to the same layer fully resident."""
    wl = gen.Workload("allcold", 4096, 2048, 384, 6, 8, n_hot=0, zipf=True)
    host = HostBuffer(384 * gen.expert_bytes(wl.hidden, wl.inter))
    try:
        fill_host_experts(host, wl.seed, 0, range(384), wl.hidden, wl.inter)
        for T in (1, 8, 40):
            L = Layer(wl, T=T, hot=[], host=host)
            assert L.n_hot == 0 and L.n_cold == 384
            L.scratch.fill_(0xEE)
            out = L.forward()
            torch.cuda.synchronize()
            ids = L.ids.cpu().numpy()
            ref = oracle_out(L)
            assert np.array_equal(ids, ref["ids"])
            err = check_out(out.cpu().numpy(), ref["out"])
            picked = set(np.unique(ids).tolist())
            scratch = L.scratch.cpu().numpy()
            hb = host.np.reshape(384, L.B)
            for e in range(384):
                s = -int(L.slot_np[e]) - 1
                if e in picked:
                    assert np.array_equal(scratch[s], hb[s]), (T, e)
                else:
                    assert scratch[s, 0] == 0xEE and np.all(scratch[s] == 0xEE), (T, e)
            print(f"no resident expert, T={T}: {len(picked)} experts gathered, max err / RMS = {err:.2e}",
                  flush=True)
            if T == 8:
                R = Layer(wl, T=T, all_hot=True)
                b = R.forward()
                torch.cuda.synchronize()
                assert torch.equal(R.ids, L.ids)
                assert torch.equal(out, b), "all-cold and all-resident outputs differ"
                del R, b
            del L, out
            torch.cuda.empty_cache()
    finally:
        host.close()


def _permuted_run(L, perm):
    """The layer with expert e relabelled perm[e]: router row, bias and
    residency entry move with the label; the bytes stay where they are."""
    inv = np.argsort(perm)
    wr = torch.from_numpy(np.ascontiguousarray(L.wr_np[inv])).cuda()
    bias = torch.from_numpy(np.ascontiguousarray(L.bias_np[inv])).cuda() if L.bias_np is not None else None
    slot = torch.from_numpy(np.ascontiguousarray(L.slot_np[inv])).cuda()
    r = moe.residency(slot, L.hot_base if L.n_hot else None, L.host.dev if L.host else None,
                      L.scratch if L.scratch is not None else None, L.n_hot, L.n_cold)
    ids = torch.empty_like(L.ids)
    w = torch.empty_like(L.w)
    out = torch.empty_like(L.out)
    ws = torch.empty_like(L.ws)
    moe.moe_layer_forward(L.shape, L.x, wr, bias, True, r, ids, w, out, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w, out


@pytest.mark.parametrize("T,n_hot", [(1, None), (3, None), (8, 40), (32, 40), (40, None), (700, None)])
def test_label_permutation(T, n_hot):
    """ids map through the relabelling; weights and outputs keep their bits
    (T=1: per-block selection; 3, 8, 32: block grouping, with cold experts at
    8 and 32; 40 and 700: the grouped GEMM with one and several token tiles)."""
    wl = gen.Workload("perm", 512, 256, 64, 6, T, n_hot=n_hot, zipf=False, seed=5)
    hot = sorted(np.random.default_rng(1).choice(64, n_hot, replace=False).tolist()) if n_hot else None
    L = Layer(wl, hot=hot)
    try:
        a = L.forward()
        torch.cuda.synchronize()
        perm = np.random.default_rng(T).permutation(L.E)
        ids_p, w_p, out_p = _permuted_run(L, perm)
        assert np.array_equal(ids_p, perm[L.ids.cpu().numpy()])
        assert torch.equal(w_p, L.w)
        assert torch.equal(out_p, a), "relabelling the experts changed the output bits"
    finally:
        L.close()


@pytest.mark.parametrize("T", [1, 5, 32, 40, 700])
def test_identical_experts_give_one_expert(T):
    """Every expert's bytes equal: with renormalised weights the layer is one
    expert's FFN on each token, whichever experts the router picks."""
    wl = gen.Workload("same", 512, 256, 64, 6, T, seed=9)
    L = Layer(wl)
    first = L.hot_base[0].clone()
    L.hot_base.copy_(first.expand_as(L.hot_base))
    out = L.forward()
    torch.cuda.synchronize()
    b0 = gen.expert_blob(wl.seed, 0, 0, wl.hidden, wl.inter)
    w13, w2 = oblob.weights(b0, wl.hidden, wl.inter)
    want = offn.expert_ffn(oroute.bf16_bits_to_f32(L.x_np), w13, w2)
    from oracle import layer as olayer
    err = olayer.max_err_over_rms(out.cpu().numpy(), want)
    assert err <= TIGHT, err
    assert len(np.unique(L.ids.cpu().numpy())) > 1


def test_scratch_poisoned_between_stacked_layers():
    """Four layers at the decode shape share one scratch, with many cold picks
    (cold experts' bias raised by 3): run in order with the scratch poisoned
    before each layer, every output equals the same layer fully resident, bit
    for bit, and each layer's gathered slots hold its own bytes."""
    wl = gen.workload("hotcold8")
    cal = gen.load_calibration()
    scratch = torch.empty((wl.n_cold, gen.expert_bytes(wl.hidden, wl.inter)), dtype=torch.uint8, device="cuda")
    layers, twins = [], []
    try:
        for l in range(4):
            L = Layer(wl, layer=l, T=32, scratch=scratch, cal=cal)
            R = Layer(wl, layer=l, T=32, all_hot=True, cal=cal)
            for X in (L, R):
                X.bias_np = X.bias_np.copy()
                X.bias_np[L.cold] += np.float32(3.0)
                X.bias.copy_(torch.from_numpy(X.bias_np))
            layers.append(L)
            twins.append(R)
        for l, (L, R) in enumerate(zip(layers, twins)):
            scratch.fill_(0x21 + l)
            a = L.forward()
            b = R.forward()
            torch.cuda.synchronize()
            assert torch.equal(L.ids, R.ids)
            assert torch.equal(a, b), f"layer {l}: output differs from the resident layer"
            ids = L.ids.cpu().numpy()
            pc = ogather.picked_cold(ids, L.slot_np)
            assert len(pc) >= 3
            sc = scratch.cpu().numpy()
            hb = L.host.np.reshape(L.n_cold, L.B)
            rows = {-int(L.slot_np[e]) - 1 for e in pc}
            for s in range(L.n_cold):
                if s in rows:
                    assert np.array_equal(sc[s], hb[s]), (l, s)
                else:
                    assert np.all(sc[s] == 0x21 + l), (l, s)
    finally:
        for L in layers:
            L.close()
