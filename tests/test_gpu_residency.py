"""Adaptive residency through the C ABI: pick counts, the byte-audit
fingerprint, and swaps between the HBM pool and the pinned host pool (the
gracetier write-up: the manager of section 1, the 3.0 hysteresis of section
3, the audit and the unchanged answers of section 4).

Bars: counts, fingerprints and the moved bytes bit-exact against the oracle;
every expert found intact at its new home (fingerprints equal to the boot
ones, 0 mismatches); layer outputs bit-identical before and after any swap
and to every expert resident, and within 1e-3 x RMS of the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from oracle import layer as olayer  # noqa: E402
from oracle import residency as ores  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_setup import Layer  # noqa: E402

TIGHT = 1e-3


def fingerprints(L, experts):
    e = torch.tensor(list(experts), dtype=torch.int32, device="cuda")
    out = torch.empty(e.numel(), dtype=torch.int64, device="cuda")
    moe.moe_fingerprint(L.shape, L.residency, e, out)
    torch.cuda.synchronize()
    return [int(v) % 2**64 for v in out.cpu().numpy().view(np.uint64)]


@pytest.mark.parametrize("T", [0, 1, 8, 1000, 5000])
def test_count_picks(T):
    E, k = 384, 6
    s = moe.shape(4096, 2048, E, k)
    rng = np.random.default_rng(T)
    counts = torch.full((E,), 7, dtype=torch.int32, device="cuda")
    ids_np = rng.integers(-3, E + 3, (max(T, 1), k)).astype(np.int32)[:T]
    ids = torch.from_numpy(ids_np).to("cuda")
    moe.moe_count_picks(s, ids, counts, clear=True)
    torch.cuda.synchronize()
    want = ores.count_picks(ids_np, E)
    assert np.array_equal(counts.cpu().numpy(), want)
    moe.moe_count_picks(s, ids, counts, clear=False)       # accumulates
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), 2 * want)


def test_fingerprint_matches_oracle():
    wl = gen.workload("hotcold8")
    L = Layer(wl, T=1)
    try:
        sample = L.hot[:3] + L.hot[-2:] + L.cold[:3] + L.cold[-2:]
        got = fingerprints(L, sample + [-1, L.E])
        for e, fp in zip(sample, got):
            assert fp == ores.fingerprint(L.blob(e)), e
        assert got[-2:] == [0, 0]      # ids outside [0, E)
    finally:
        L.close()


def boost(L, experts, delta):
    bias = L.bias_np.copy()
    bias[list(experts)] += np.float32(delta)
    L.bias_np = bias
    L.bias.copy_(torch.from_numpy(bias))


def audit(L, boot, moved, rng, n_random=64):
    """Fingerprint every moved expert plus n_random others where they now live."""
    others = [e for e in range(L.E) if e not in moved]
    sample = sorted(set(moved) | set(rng.choice(others, min(n_random, len(others)), replace=False).tolist()))
    got = fingerprints(L, sample)
    return sum(1 for e, fp in zip(sample, got) if fp != boot[e])


def test_swap_moves_bytes_and_keeps_outputs():
    wl = gen.workload("hotcold8")
    L = Layer(wl, T=8)
    hot = Layer(wl, T=8, all_hot=True)
    rng = np.random.default_rng(5)
    try:
        promote = L.cold[:5]
        boost(L, promote, 3.0)
        hot.bias_np = L.bias_np
        hot.bias.copy_(L.bias)
        boot = fingerprints(L, range(L.E))
        out0 = L.forward().clone()
        ref = hot.forward().clone()
        torch.cuda.synchronize()
        ids0 = L.ids.clone()
        assert torch.equal(out0, ref)

        # one manager tick with crafted counts: the five boosted cold experts
        # are picked often, everything else rarely
        slot = L.slot_np.copy()
        score = np.zeros(L.E)
        counts = np.ones(L.E, dtype=np.int32)
        counts[promote] = 50
        pairs = moe.moe_residency_plan(L.shape, slot, L.n_hot, L.n_cold, score, counts, 1.0, 3.0, 1.0, 64)
        o_pairs, o_slot, _ = ores.manager_tick(L.slot_np, np.zeros(L.E), counts, 1.0, 3.0, 1.0, 64)
        assert [tuple(p) for p in pairs.tolist()] == o_pairs and len(o_pairs) == 5
        old = L.slot_np.copy()
        L.scratch.fill_(0xEE)
        moe.moe_residency_swap(L.shape, L.residency, pairs)
        torch.cuda.synchronize()
        assert np.array_equal(L.slot.cpu().numpy(), slot)
        L.slot_np = slot

        # bytes at their new homes (against the oracle's move of the pools)
        host_pool = L.host.np.reshape(L.n_cold, L.B)
        for c, h in o_pairs:
            assert np.array_equal(L.hot_base[int(old[h])].cpu().numpy(), L.blob(c))
            assert np.array_equal(host_pool[-old[c] - 1], L.blob(h))
        # audit: every expert where it now lives
        assert fingerprints(L, range(L.E)) == boot
        assert audit(L, boot, [e for p in o_pairs for e in p], rng) == 0

        # same tokens, new map: same ids and bit-identical output; nothing
        # promoted is gathered any more
        L.scratch.fill_(0xEE)
        out1 = L.forward().clone()
        torch.cuda.synchronize()
        assert torch.equal(L.ids, ids0)
        assert torch.equal(out1, out0)
        picked = set(ids0.cpu().numpy().reshape(-1).tolist())
        for c, h in o_pairs:
            # c's old cold slot now belongs to h: gathered only if h was picked
            row = L.scratch[int(-old[c] - 1)].cpu().numpy()
            if h in picked:
                assert np.array_equal(row, L.blob(h))
            else:
                assert np.all(row == 0xEE)

        # and back again: swap the five out with the rule's own numbers
        counts = np.ones(L.E, dtype=np.int32)
        counts[[h for _, h in o_pairs]] = 500
        counts[promote] = 0
        pairs2 = moe.moe_residency_plan(L.shape, slot, L.n_hot, L.n_cold, np.zeros(L.E), counts, 1.0, 3.0, 1.0, 64)
        assert sorted(pairs2[:, 0].tolist()) == sorted(h for _, h in o_pairs)
        moe.moe_residency_swap(L.shape, L.residency, pairs2)
        torch.cuda.synchronize()
        assert np.array_equal(L.slot.cpu().numpy(), slot)
        L.slot_np = slot
        assert fingerprints(L, range(L.E)) == boot
        out2 = L.forward()
        torch.cuda.synchronize()
        assert torch.equal(out2, out0)
        rows = [0, 7]
        o = olayer.layer_forward(L.x_np[rows], L.wr_np, L.bias_np, L.blob, L.H, L.I, L.k)
        assert np.array_equal(L.ids.cpu().numpy()[rows], o["ids"])
        assert olayer.max_err_over_rms(out2.cpu().numpy()[rows], o["out"]) <= TIGHT
    finally:
        L.close()
        hot.close()


def test_manager_ticks_on_routed_traffic():
    """Ticks driven by the layer's own pick counts (moe_count_picks) on
    shifting traffic: after every tick the table is valid, every moved expert
    and 64 others audit clean, and the layer output equals every expert
    resident bit for bit."""
    wl = gen.workload("hotcold8")
    L = Layer(wl, T=32)
    hot = Layer(wl, T=32, all_hot=True)
    rng = np.random.default_rng(11)
    counts = torch.zeros(L.E, dtype=torch.int32, device="cuda")
    try:
        boot = fingerprints(L, range(L.E))
        slot = L.slot_np.copy()
        score = np.zeros(L.E)
        moved_total = 0
        for tick in range(4):
            shift = rng.choice(L.cold, 12, replace=False)
            boost(L, shift, 2.0)
            hot.bias_np = L.bias_np
            hot.bias.copy_(L.bias)
            moe.moe_count_picks(L.shape, None, counts, clear=True)
            for _ in range(3):
                out = L.forward()
                moe.moe_count_picks(L.shape, L.ids, counts)
            ref = hot.forward()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), tick
            c = counts.cpu().numpy()
            pairs = moe.moe_residency_plan(L.shape, slot, L.n_hot, L.n_cold, score, c, 0.5, 3.0, 1.0, 16)
            moe.moe_residency_swap(L.shape, L.residency, pairs)
            torch.cuda.synchronize()
            assert np.array_equal(L.slot.cpu().numpy(), slot)
            L.slot_np = slot.copy()
            moe.moe_residency_check(L.shape, slot, L.n_hot, L.n_cold)
            moved = [int(e) for e in pairs.reshape(-1)]
            moved_total += len(pairs)
            assert audit(L, boot, moved, rng) == 0, tick
        assert moved_total > 0
        out = L.forward()
        ref = hot.forward()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert fingerprints(L, range(L.E)) == boot
    finally:
        L.close()
        hot.close()


def test_swap_rejects_direct_read_and_bad_pairs():
    wl = gen.workload("hotcold8")
    d = Layer(wl, T=1, direct=True)
    try:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_residency_swap(d.shape, d.residency, [[d.cold[0], d.hot[0]]])
        assert ei.value.status == moe.MOE_ERR_BAD_RESIDENCY
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_residency_swap(d.shape, d.residency, [[d.cold[0], d.hot[0]], [d.cold[1], d.hot[0]]])
        assert ei.value.status in (moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_BAD_RESIDENCY)
    finally:
        d.close()
    L = Layer(wl, T=1)
    try:
        before = L.slot.clone()
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_residency_swap(L.shape, L.residency, [[L.cold[0], L.hot[0]], [L.cold[1], L.hot[0]]])
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
        # a pair the table does not show as (cold, hot) is left alone on the device
        moe.moe_residency_swap(L.shape, L.residency, [[L.hot[1], L.cold[2]]])
        torch.cuda.synchronize()
        assert torch.equal(L.slot, before)
    finally:
        L.close()


def test_swap_of_the_most_pairs_at_once():
    """MOE_MAX_SWAPS pairs in one call (the grid's pair axis at its largest):
    table, bytes (audited) and outputs as the oracle's moves say."""
    wl = gen.workload("hotcold8")
    L = Layer(wl, T=8)
    try:
        boot = fingerprints(L, range(L.E))
        out0 = L.forward().clone()
        n = moe.MOE_MAX_SWAPS
        pairs = np.array(list(zip(L.cold[:n], L.hot[-n:])), dtype=np.int32)
        want = L.slot_np.copy()
        for c, h in pairs:
            want[c], want[h] = want[h], want[c]
        moe.moe_residency_swap(L.shape, L.residency, pairs)
        torch.cuda.synchronize()
        assert np.array_equal(L.slot.cpu().numpy(), want)
        L.slot_np = want
        assert fingerprints(L, range(L.E)) == boot
        out1 = L.forward()
        torch.cuda.synchronize()
        assert torch.equal(out1, out0)
    finally:
        L.close()


def test_fingerprint_past_the_grid_row_limit():
    """More fingerprints than one launch's grid rows (65,535): every id,
    repeated, gets its expert's value; out-of-range ids give 0."""
    E = 8
    s = moe.shape(256, 128, E, 2)
    B = moe.moe_expert_bytes(s)
    rng = np.random.default_rng(3)
    blobs = rng.integers(0, 256, (E, B), dtype=np.uint8)
    hot = torch.from_numpy(blobs[:6].copy()).cuda()
    from tests.gpu_setup import HostBuffer
    host = HostBuffer(2 * B)
    try:
        host.np[:] = blobs[6:].reshape(-1)
        scratch = torch.empty((2, B), dtype=torch.uint8, device="cuda")
        slot = torch.tensor([0, 1, 2, 3, 4, 5, -1, -2], dtype=torch.int32, device="cuda")
        r = moe.residency(slot, hot, host.dev, scratch, 6, 2)
        n = 70000
        ids_np = rng.integers(-1, E + 1, n).astype(np.int32)
        ids = torch.from_numpy(ids_np).cuda()
        out = torch.empty(n, dtype=torch.int64, device="cuda")
        moe.moe_fingerprint(s, r, ids, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint64)
        ref = [ores.fingerprint(blobs[e]) for e in range(E)]
        for i in range(n):
            e = ids_np[i]
            assert int(got[i]) == (ref[e] if 0 <= e < E else 0), i
    finally:
        host.close()
