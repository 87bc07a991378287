"""Parity of the HIP path (through the C ABI) against the CPU oracle.

The bars and the index rules R1-R3 are stated in tests/gpu_checks.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from oracle import gather as ogather  # noqa: E402
from oracle import route as oroute  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_checks import TIGHT, check_out, check_route, oracle_out, route_on_gpu  # noqa: E402
from tests.gpu_setup import Layer, Stack  # noqa: E402


# ------------------------------------------------------------------------------
def test_device_generator_matches_cpu():
    H, I = 4096, 2048
    out = torch.empty((3, gen.expert_bytes(H, I)), dtype=torch.uint8, device="cuda")
    gen.fill_expert_blobs_device(out, 0, 5, [0, 200, 383], H, I)
    host = out.cpu().numpy()
    for i, e in enumerate((0, 200, 383)):
        assert np.array_equal(host[i], gen.expert_blob(0, 5, e, H, I)), e


@pytest.mark.parametrize("T", [4, 1, 3, 17, 37, 300, 1000])
def test_tiny_layer(T):
    """T <= 32: decode kernels; T > 32 at this shape (H=256): one-wave kernels."""
    L = Layer(gen.workload("tiny"), T=T)
    ids_g, w_g, z_g = route_on_gpu(L)
    check_route(L, ids_g, w_g, z_g)
    out = L.forward()
    torch.cuda.synchronize()
    assert np.array_equal(L.ids.cpu().numpy(), ids_g)
    ref = oracle_out(L)
    assert np.array_equal(ref["ids"], ids_g)
    check_out(out.cpu().numpy(), ref["out"])


def test_tiny_unnormalised_weights():
    L = Layer(gen.workload("tiny"), T=9)
    ids_g, w_g, z_g = route_on_gpu(L, renorm=False)
    check_route(L, ids_g, w_g, z_g, renorm=False)
    assert np.all(w_g.sum(axis=1) < 1.0 + 1e-6)


def test_decode1_layer():
    L = Layer(gen.workload("decode1"))
    ids_g, w_g, z_g = route_on_gpu(L)
    check_route(L, ids_g, w_g, z_g)
    out = L.forward()
    torch.cuda.synchronize()
    ref = oracle_out(L)
    assert np.array_equal(L.ids.cpu().numpy(), ref["ids"])
    err = check_out(out.cpu().numpy(), ref["out"])
    print(f"decode1: max err / RMS = {err:.2e}")


def test_hotcold8_layer_gather_and_pick_set():
    L = Layer(gen.workload("hotcold8"))
    try:
        L.scratch.fill_(0xEE)
        ids_g, w_g, z_g = route_on_gpu(L)
        check_route(L, ids_g, w_g, z_g)
        # pick set, bit exact
        counts = torch.empty(L.E, dtype=torch.int32, device="cuda")
        cold = torch.empty(L.E + 1, dtype=torch.int32, device="cuda")
        ids_t = torch.from_numpy(ids_g).cuda()
        moe.moe_pick_set(L.shape, ids_t, L.slot, L.n_hot, L.n_cold, counts, cold, L.ws)
        torch.cuda.synchronize()
        assert np.array_equal(counts.cpu().numpy(), ogather.pick_counts(ids_g, L.E))
        pc = ogather.picked_cold(ids_g, L.slot_np)
        c = cold.cpu().numpy()
        assert c[0] == len(pc) and np.array_equal(c[1:1 + len(pc)], pc)
        # layer, with its gather
        out = L.forward()
        torch.cuda.synchronize()
        ref = oracle_out(L)
        assert np.array_equal(L.ids.cpu().numpy(), ref["ids"])
        check_out(out.cpu().numpy(), ref["out"])
        # gathered bytes == host bytes; unpicked slots untouched
        B = L.B
        host = L.host.np.reshape(L.n_cold, B)
        want_rows = {-int(L.slot_np[e]) - 1 for e in pc}
        scratch = L.scratch.cpu().numpy()
        for cs in range(L.n_cold):
            if cs in want_rows:
                assert np.array_equal(scratch[cs], host[cs]), cs
            else:
                assert np.all(scratch[cs] == 0xEE), cs
        print(f"hotcold8: distinct experts {len(np.unique(ids_g))}, picked cold {len(pc)}")
    finally:
        L.close()


def test_all_hot_equals_mixed_bitwise():
    wl = gen.workload("hotcold8")
    mixed = Layer(wl)
    hot = Layer(wl, all_hot=True)
    try:
        a = mixed.forward()
        b = hot.forward()
        torch.cuda.synchronize()
        assert torch.equal(mixed.ids, hot.ids)
        assert torch.equal(a, b), "hot/cold placement changed the output bits"
    finally:
        mixed.close()


def boost_cold(L, delta):
    """Raise the router bias of L's cold experts by delta (oracle and GPU)."""
    L.bias_np = L.bias_np.copy()
    L.bias_np[L.cold] += np.float32(delta)
    L.bias.copy_(torch.from_numpy(L.bias_np))


@pytest.mark.parametrize("T,delta", [(32, 3.0), (5, 3.0), (32, 0.0), (1, 3.0), (1, 40.0), (8, 40.0),
                                     (2, 3.0), (4, 3.0), (4, 40.0)])
def test_decode_cold_picks_overlapped(T, delta):
    """Decode layer with many picked cold experts: the gather runs on the side
    stream while the hot experts' FFN runs; ids, gathered bytes and outputs
    must be as with every expert resident."""
    wl = gen.workload("hotcold8")
    L = Layer(wl, T=T)
    hot = Layer(wl, T=T, all_hot=True)
    try:
        boost_cold(L, delta)
        hot.bias_np = L.bias_np
        hot.bias.copy_(L.bias)
        L.scratch.fill_(0xEE)
        a = L.forward()
        b = hot.forward()
        torch.cuda.synchronize()
        ids = L.ids.cpu().numpy()
        pc = ogather.picked_cold(ids, L.slot_np)
        print(f"T={T} delta={delta}: picked cold {len(pc)}", flush=True)
        if delta > 0:
            assert len(pc) >= min(3, T)
        if delta >= 40:   # every pick cold: the HBM-resident part has nothing to do
            assert len(pc) == len(np.unique(ids))
        assert torch.equal(L.ids, hot.ids)
        assert torch.equal(a, b), "hot/cold placement changed the output bits"
        host = L.host.np.reshape(L.n_cold, L.B)
        scratch = L.scratch.cpu().numpy()
        want_rows = {-int(L.slot_np[e]) - 1 for e in pc}
        for cs in range(L.n_cold):
            if cs in want_rows:
                assert np.array_equal(scratch[cs], host[cs]), cs
            else:
                assert np.all(scratch[cs] == 0xEE), cs
        rows = sorted({0, T // 2, T - 1})
        ref = oracle_out(L, rows=rows)
        assert np.array_equal(ids[rows], ref["ids"])
        check_out(a.cpu().numpy()[rows], ref["out"])
    finally:
        L.close()
        hot.close()


@pytest.mark.parametrize("m", [1, 5, 129])
def test_forced_cold_gather(m):
    """ids crafted to pick exactly m distinct cold experts (plus hot ones)."""
    L = Layer(gen.workload("hotcold8"))
    try:
        L.scratch.fill_(0x5A)
        rng = np.random.default_rng(m)
        cold_pick = sorted(rng.choice(L.cold, size=m, replace=False).tolist())
        T = max(1, -(-m // L.k))
        ids = np.array(L.hot[: T * L.k], dtype=np.int32).reshape(T, L.k)
        flat = ids.reshape(-1)
        flat[:m] = cold_pick
        ids_t = torch.from_numpy(ids).cuda()
        ws = torch.empty(moe.moe_workspace_bytes(L.shape, T), dtype=torch.uint8, device="cuda")
        moe.moe_gather_cold(L.shape, ids_t, L.residency, ws)
        torch.cuda.synchronize()
        scratch = L.scratch.cpu().numpy()
        want = ogather.gather_cold(ids, L.slot_np, L.host.np.reshape(L.n_cold, L.B),
                                   np.full((L.n_cold, L.B), 0x5A, dtype=np.uint8))
        assert np.array_equal(scratch, want)
    finally:
        L.close()


def test_gemm_hot_cold_equals_all_hot_and_oracle():
    """Grouped-GEMM path with a hot/cold split: bit-identical to the all-hot
    run, and within the bars against the oracle.  48 experts over 1500 tokens
    (~187 pairs per expert: one or two token tiles)."""
    wl = gen.Workload("gemm_hc", 512, 256, 48, 6, 1500, n_hot=30)
    hot = list(range(0, 48, 2)) + [1, 3, 5, 7, 9, 11]
    mixed = Layer(wl, hot=hot)
    allhot = Layer(wl, all_hot=True)
    try:
        mixed.scratch.fill_(0xEE)
        a = mixed.forward()
        b = allhot.forward()
        torch.cuda.synchronize()
        assert torch.equal(mixed.ids, allhot.ids)
        assert torch.equal(a, b), "hot/cold placement changed the output bits"
        ref = oracle_out(mixed)
        assert np.array_equal(mixed.ids.cpu().numpy(), ref["ids"])
        check_out(a.cpu().numpy(), ref["out"])
    finally:
        mixed.close()


@pytest.mark.parametrize("E,k,T", [(64, 2, 2000), (64, 2, 3000), (32, 4, 1100), (16, 3, 700)])
def test_gemm_tile_shapes(E, k, T):
    """Grouped-GEMM path (H=512, I=256) at token counts per expert that give
    every number of 32-token column tiles (1..5) and ragged last tiles."""
    wl = gen.Workload("gemm_shapes", 512, 256, E, k, T, seed=E + k)
    L = Layer(wl)
    out = L.forward()
    torch.cuda.synchronize()
    ids = L.ids.cpu().numpy()
    counts = np.bincount(ids.reshape(-1), minlength=E)
    tiles = np.concatenate([[min(160, c - p) for p in range(0, c, 160)] for c in counts if c > 0])
    print(f"E={E} k={k} T={T}: column tiles per token tile {sorted(set(((tiles + 31) // 32).tolist()))}")
    ref = oracle_out(L)
    assert np.array_equal(ids, ref["ids"])
    check_out(out.cpu().numpy(), ref["out"])


def test_gemm_rows_over_six_decades():
    """Grouped-GEMM path with each token scaled by 10^u, u uniform in [-3, 3]:
    every output row stays within the tight bound of its own RMS, so the
    GEMMs keep a relative precision per token whatever its magnitude (h's
    e4m3 terms take their scales per 32 columns of a token; silu of a large
    negative gate underflows to -0 on both sides).  The routing margins of
    these seeded tokens are at least 9e-5 of their largest logit, far above
    fp32 rounding, so the ids must match exactly."""
    wl = gen.Workload("gemm_range", 512, 256, 16, 2, 700, seed=7)
    x = oroute.bf16_bits_to_f32(gen.tokens_bf16(wl.seed, 0, wl.tokens, wl.hidden)).astype(np.float32)
    s = (10.0 ** np.random.default_rng(3).uniform(-3, 3, size=(wl.tokens, 1))).astype(np.float32)
    L = Layer(wl, x_np=gen.bf16_round_bits(x * s))
    try:
        out = L.forward().cpu().numpy()
        ref = oracle_out(L)
        assert np.array_equal(L.ids.cpu().numpy(), ref["ids"])
        got, want = out.astype(np.float64), ref["out"].astype(np.float64)
        row_rms = np.sqrt(np.mean(want * want, axis=1))
        err = np.max(np.abs(got - want), axis=1) / row_rms
        print(f"rows over six decades: row RMS {row_rms.min():.2e}..{row_rms.max():.2e}, "
              f"max row err / row RMS = {err.max():.2e}")
        assert err.max() <= TIGHT, err.max()
    finally:
        L.close()


def test_gemm_max_experts_and_k():
    """Grouped-GEMM path at the ABI's largest expert count and top-k (E =
    1024, k = 32; 300 tokens, H = 512): every expert is picked, with at most
    21 pairs, so the tile list holds 1024 one-column-tile tiles (distinct
    index up to 1023 in its 10-bit field); the router GEMM runs 16 expert
    tiles and the top-k its widest form.  Routing by R1-R3, outputs within the
    bars (the smallest oracle margin, 4.9e-5, is far above the fp32 logit
    error at this size, so the ids must match exactly)."""
    wl = gen.Workload("gemm_maxek", 512, 256, 1024, 32, 300, seed=11)
    L = Layer(wl)
    try:
        ids_g, w_g, z_g = route_on_gpu(L)
        check_route(L, ids_g, w_g, z_g)
        out = L.forward()
        torch.cuda.synchronize()
        ref = oracle_out(L)
        assert np.array_equal(L.ids.cpu().numpy(), ref["ids"])
        assert len(np.unique(ref["ids"])) == 1024
        check_out(out.cpu().numpy(), ref["out"])
    finally:
        L.close()


def test_wave_path_for_unaligned_hidden():
    """T > 32 with H not a multiple of 256 runs the one-wave kernels."""
    wl = gen.Workload("h384", 384, 256, 16, 4, 48, seed=3)
    L = Layer(wl)
    out = L.forward()
    torch.cuda.synchronize()
    ref = oracle_out(L)
    assert np.array_equal(L.ids.cpu().numpy(), ref["ids"])
    check_out(out.cpu().numpy(), ref["out"])


@pytest.mark.timeout(900)
def test_step40_full_size():
    """The 40-layer decode step at full size: 40 x (255 hot in HBM, 129 cold in
    pinned host memory), one shared 129-slot scratch, batch 32, run in layer
    order on one stream.  Checks: routing of every layer (R1-R3 against the
    oracle); outputs of sampled layers and tokens; and the shared scratch after
    the step - each slot holds the bytes of the last layer that picked the
    cold expert mapped to it, and a slot no layer picked is untouched; then
    the step once more with the scratch poisoned before every layer gives the
    same outputs bit for bit."""
    wl = gen.workload("step40")
    B = gen.expert_bytes(wl.hidden, wl.inter)
    need = (wl.layers * wl.n_hot + wl.n_cold) * B
    if torch.cuda.mem_get_info()[0] < need * 1.05:
        pytest.skip("not enough device memory for the 40-layer step")
    try:
        S = Stack(wl)
    except moe.MoeError as e:
        pytest.skip(f"pinned host memory for the 40 cold pools is not available here ({e})")
    try:
        S.scratch.fill_(0xEE)
        S.forward()
        torch.cuda.synchronize()
        picks = []
        for L in S.layers:
            ids_g, w_g, z_g = route_on_gpu(L)
            assert np.array_equal(L.ids.cpu().numpy(), ids_g)
            check_route(L, ids_g, w_g, z_g)
            picks.append(ids_g)
        rows = np.array([0, 31])
        for li in (0, 39):
            L = S.layers[li]
            ref = oracle_out(L, rows)
            check_out(L.out.cpu().numpy()[rows], ref["out"])
        # shared scratch: last writer per slot
        scratch = S.scratch.cpu().numpy()
        last = {}
        for li, L in enumerate(S.layers):
            for e in ogather.picked_cold(picks[li], L.slot_np):
                last[-int(L.slot_np[e]) - 1] = li
        for cs in range(wl.n_cold):
            if cs in last:
                L = S.layers[last[cs]]
                assert np.array_equal(scratch[cs], L.host.np[cs * B:(cs + 1) * B]), (cs, last[cs])
            else:
                assert np.all(scratch[cs] == 0xEE), cs
        # the same step again, layer by layer, with the scratch poisoned
        # before every layer: each layer reads only slots it gathered itself,
        # so every output keeps its bits
        first = [L.out.clone() for L in S.layers]
        for li, L in enumerate(S.layers):
            S.scratch.fill_(0x11 * (li % 15 + 1))
            L.forward()
        torch.cuda.synchronize()
        for li, L in enumerate(S.layers):
            assert torch.equal(L.out, first[li]), f"layer {li}: a stale scratch slot reached the output"
        n_cold = [len(ogather.picked_cold(p, L.slot_np)) for p, L in zip(picks, S.layers)]
        print(f"step40: distinct experts per layer {np.mean([len(np.unique(p)) for p in picks]):.1f}, "
              f"picked cold per layer {np.mean(n_cold):.2f}, scratch slots written {len(last)}")
    finally:
        S.close()


def test_max_experts_and_k():
    wl = gen.Workload("maxek", 128, 128, 1024, 32, 5)
    L = Layer(wl)
    ids_g, w_g, z_g = route_on_gpu(L)
    check_route(L, ids_g, w_g, z_g)
    out = L.forward()
    torch.cuda.synchronize()
    check_out(out.cpu().numpy(), oracle_out(L)["out"])


@pytest.mark.parametrize("cold", [False, True])
def test_many_experts_few_pairs(cold):
    """E = 1024 with 8 pairs (the one-token launch sequences' limit) and a
    small hidden size: the decode launches whose blocks would hold fewer
    threads than half the residency entries take the grouped path instead;
    routing and outputs as the oracle's, hot/cold bit-identical to all
    resident."""
    wl = gen.Workload("manyE", 128, 128, 1024, 2, 4)
    hot = list(range(0, 1024, 2)) if cold else None
    L = Layer(wl, hot=hot)
    ref_layer = Layer(wl) if cold else None
    try:
        ids_g, w_g, z_g = route_on_gpu(L)
        check_route(L, ids_g, w_g, z_g)
        out = L.forward()
        torch.cuda.synchronize()
        check_out(out.cpu().numpy(), oracle_out(L)["out"])
        if cold:
            assert len(ogather.picked_cold(L.ids.cpu().numpy(), L.slot_np)) > 0
            ref = ref_layer.forward()
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
    finally:
        L.close()
        if ref_layer is not None:
            ref_layer.close()


def test_k1_single_expert():
    wl = gen.Workload("k1", 256, 128, 8, 1, 6)
    L = Layer(wl)
    out = L.forward()
    torch.cuda.synchronize()
    assert np.all(L.w.cpu().numpy() == 1.0)
    check_out(out.cpu().numpy(), oracle_out(L)["out"])


def test_bf16_output_is_rounded_fp32():
    L = Layer(gen.workload("tiny"), T=7)
    f = L.forward().clone()
    b = L.forward(out_bf16=True)
    torch.cuda.synchronize()
    assert torch.equal(b, f.to(torch.bfloat16))


@pytest.mark.parametrize("T,bad_pos", [(6, [(1, 0), (3, 1)]), (2, [(0, 1), (1, 0)]), (20, [(0, 1), (19, 0)])])
def test_invalid_ids_contribute_zero(T, bad_pos):
    """T=2 (4 pairs) runs the fused down + combine kernel, T=6 the down blocks
    that combine their row tiles themselves, T=20 the down blocks and then
    the combine launch."""
    L = Layer(gen.workload("tiny"), T=T)
    ids_g, w_g, _ = route_on_gpu(L)
    bad = ids_g.copy()
    bad[bad_pos[0]] = -1
    bad[bad_pos[1]] = L.E
    out = torch.empty((L.T, L.H), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(L.shape, L.x, torch.from_numpy(bad).cuda(), torch.from_numpy(w_g).cuda(), L.residency,
                       out, L.ws)
    torch.cuda.synchronize()
    ref = oracle_out(L)
    y = ref["y"].copy()
    y[bad_pos[0]] = 0
    y[bad_pos[1]] = 0
    from oracle.ffn import combine
    want = combine(w_g, y)
    check_out(out.cpu().numpy(), want)


@pytest.mark.parametrize("T", [1, 6, 20])
def test_unusable_residency_entry_contributes_zero(T):
    """A device residency entry outside [0, n_hot) makes that expert's pairs
    contribute zero (fused down + combine at T=1, down blocks that combine
    at T=6, down blocks and a combine launch at T=20)."""
    L = Layer(gen.workload("tiny"), T=T)
    ids_g, w_g, _ = route_on_gpu(L)
    e_bad = int(ids_g[0, 0])
    slot = L.slot_np.copy()
    slot[e_bad] = L.n_hot + 7
    r = moe.residency(torch.from_numpy(slot).cuda(), L.hot_base, None, None, L.n_hot, 0)
    out = torch.empty((L.T, L.H), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(L.shape, L.x, torch.from_numpy(ids_g).cuda(), torch.from_numpy(w_g).cuda(), r, out, L.ws)
    torch.cuda.synchronize()
    ref = oracle_out(L)
    assert np.array_equal(ids_g, ref["ids"])
    y = ref["y"].copy()
    y[ids_g == e_bad] = 0
    from oracle.ffn import combine
    check_out(out.cpu().numpy(), combine(w_g, y))


@pytest.mark.parametrize("T", [2, 6, 20])
def test_all_ids_invalid_give_zero_output(T):
    """With no valid pick there is no distinct expert, so no down block counts
    itself in: the output must still be written, as zeros, by every path
    (fused down + combine, down blocks that combine, combine launch), also
    over a workspace that the previous call left with live counters."""
    L = Layer(gen.workload("tiny"), T=T)
    ids_g, w_g, _ = route_on_gpu(L)
    out = torch.full((L.T, L.H), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(L.shape, L.x, torch.from_numpy(ids_g).cuda(), torch.from_numpy(w_g).cuda(), L.residency,
                       out, L.ws)
    bad = np.where(np.arange(ids_g.size).reshape(ids_g.shape) % 2 == 0, -1, L.E).astype(ids_g.dtype)
    moe.moe_expert_ffn(L.shape, L.x, torch.from_numpy(bad).cuda(), torch.from_numpy(w_g).cuda(), L.residency,
                       out, L.ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("mode", ["invalid_ids", "unusable_entry"])
def test_gemm_invalid_ids_and_unusable_entry(mode):
    """The grouped-GEMM path (100 tokens, H = 512): picks with an id outside
    [0, E) are left out of the grouping and of the combine; an expert whose
    residency entry is outside [0, n_hot) makes its pairs contribute zero (its
    gate/up tiles skip it, its down tiles write zeros).  Either way the
    output is the oracle's combine with those pairs' outputs set to zero."""
    wl = gen.Workload("gemm_bad", 512, 256, 16, 3, 100, seed=5)
    L = Layer(wl)
    try:
        ids_g, w_g, _ = route_on_gpu(L)
        ref = oracle_out(L)
        assert np.array_equal(ids_g, ref["ids"])
        y = ref["y"].copy()
        ids_in, r = ids_g.copy(), L.residency
        if mode == "invalid_ids":
            for t, j, v in ((0, 1, -1), (17, 0, L.E), (63, 2, -5), (99, 1, L.E + 3)):
                ids_in[t, j] = v
                y[t, j] = 0
        else:
            e_bad = int(ids_g[40, 0])
            slot = L.slot_np.copy()
            slot[e_bad] = L.n_hot + 7
            r = moe.residency(torch.from_numpy(slot).cuda(), L.hot_base, None, None, L.n_hot, 0)
            y[ids_g == e_bad] = 0
        out = torch.empty((L.T, L.H), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(L.shape, L.x, torch.from_numpy(ids_in).cuda(), torch.from_numpy(w_g).cuda(), r, out,
                           L.ws)
        torch.cuda.synchronize()
        from oracle.ffn import combine
        check_out(out.cpu().numpy(), combine(w_g, y))
    finally:
        L.close()


def test_zero_tokens_is_a_no_op():
    L = Layer(gen.workload("tiny"), T=4)
    L.out.fill_(7.0)
    x0 = L.x[:0]
    moe.moe_layer_forward(L.shape, x0, L.wr, None, True, L.residency, L.ids[:0], L.w[:0], L.out[:0], L.ws)
    torch.cuda.synchronize()
    assert torch.all(L.out == 7.0)


def test_gpu_error_paths():
    """Every bad call is rejected on the host; each also carries a second
    error (a too-small workspace size) so no launch could follow even if the
    first check misjudged."""
    import ctypes
    L = Layer(gen.workload("tiny"), T=4)
    lib = moe.lib
    host = np.zeros((4, L.H), dtype=np.uint16)       # ordinary pageable host memory
    st = lib.moe_route(ctypes.byref(L.shape), 4, host.ctypes.data, L.wr.data_ptr(), None, 1, L.ids.data_ptr(),
                       L.w.data_ptr(), None, L.ws.data_ptr(), 16, None)
    assert st == moe.MOE_ERR_NOT_DEVICE_ACCESSIBLE, moe.moe_last_error()
    st = lib.moe_route(ctypes.byref(L.shape), 4, L.x.data_ptr(), L.wr.data_ptr(), None, 1, L.ids.data_ptr(),
                       L.w.data_ptr(), None, L.ws.data_ptr(), 16, None)
    assert st == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    st = lib.moe_route(ctypes.byref(L.shape), 4, L.x.data_ptr() + 2, L.wr.data_ptr(), None, 1,
                       L.ids.data_ptr(), L.w.data_ptr(), None, L.ws.data_ptr(), 16, None)
    assert st == moe.MOE_ERR_MISALIGNED


@pytest.mark.parametrize("name,T,delta", [("tiny", 8, 0.0), ("hotcold8", 8, 0.0), ("hotcold8", 32, 3.0),
                                          ("hotcold8", 1, 3.0), ("hotcold8", 1, 0.0), ("hotcold8", 4, 3.0),
                                          ("hotcold8", 40, 3.0), ("hotcold8", 300, 0.0)])
def test_graph_replay_matches_eager(name, T, delta):
    """The layer captured in a HIP graph gives the eager result on every
    replay, with eager work and synchronisations between replays (with cold
    picks the capture holds the side-stream fork and join; from 33 tokens the
    grouping kernels and the grouped GEMMs are captured)."""
    L = Layer(gen.workload(name), T=T)
    try:
        if delta:
            boost_cold(L, delta)
        eager = L.forward().clone()
        eager_ids = L.ids.clone()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
            moe.moe_layer_forward(L.shape, L.x, L.wr, L.bias, True, L.residency, L.ids, L.w, L.out, L.ws, s)
        torch.cuda.synchronize()
        for i in range(4):
            L.out.fill_(float(i))
            L.ids.fill_(-7)
            if L.scratch is not None:
                L.scratch.fill_(0x33)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(L.ids, eager_ids), i
            assert torch.equal(L.out, eager), i
    finally:
        L.close()
