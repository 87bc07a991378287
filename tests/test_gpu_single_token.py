"""The decode path for one token's worth of pairs (T*k <= 8: gate/up tiles,
then the down projection fused with the combine) through the C ABI, against
the oracle and against itself across entry points and residencies.

Shapes beyond the tiny and decode cases, chosen so the oracle still finishes
in seconds: gate/up blocks with one and two row tiles (T = 8 at k = 1), down
K slices of one and two steps, repeated experts (fewer distinct experts than
pairs, down to 3 experts for 8 pairs), exactly eight pairs, and the selection
recomputed in every gate/up block (moe_layer_forward) or taken from the
grouping (moe_expert_ffn, and the cold part of a mixed residency)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from oracle import layer as olayer  # noqa: E402
from oracle.ffn import combine  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_setup import Layer  # noqa: E402

TOL = 2e-2
TIGHT = 1e-3

# (name, H, I, E, k, T): pairs T*k <= 8
SHAPES = [
    ("f_h1k_i512_k4_t1", 1024, 512, 16, 4, 1),    # idle down waves
    ("f_h1k_i512_k4_t2", 1024, 512, 16, 4, 2),    # 8 pairs
    ("f_h1k_i1k_k2_t3", 1024, 1024, 8, 2, 3),     # repeated experts likely
    ("f_h1k_i1k_k1_t8", 1024, 1024, 16, 1, 8),    # two row tiles per gate/up block
    ("f_h2k_i2k_k8_t1", 2048, 2048, 64, 8, 1),    # down slices of 2 steps, 8 pairs
    ("f_h1k_i512_k2_t4_e3", 1024, 512, 3, 2, 4),  # 3 experts for 8 pairs
]


def wl_of(name, H, I, E, k, T, seed=11):
    return gen.Workload(name, H, I, E, k, T, seed=seed)


def oracle_out(L):
    return olayer.layer_forward(L.x_np, L.wr_np, L.bias_np, L.blob, L.H, L.I, L.k)


def check_out(got, ref):
    err = olayer.max_err_over_rms(got, ref)
    assert err <= TOL, f"layer output error {err:.3e} x RMS exceeds the 2e-2 bar"
    assert err <= TIGHT, f"layer output error {err:.3e} x RMS above this path's arithmetic bound"
    return err


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_single_token_layer_matches_oracle(shape):
    L = Layer(wl_of(*shape))
    try:
        out = L.forward()
        torch.cuda.synchronize()
        ref = oracle_out(L)
        assert np.array_equal(L.ids.cpu().numpy(), ref["ids"])
        err = check_out(out.cpu().numpy(), ref["out"])
        print(f"{shape[0]}: distinct {len(np.unique(ref['ids']))} of {L.T * L.k} pairs, err/RMS {err:.2e}")
    finally:
        L.close()


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_single_token_expert_ffn_equals_layer_bitwise(shape):
    """The grouping-fed gate/up (moe_expert_ffn) and the selection-fed one
    (moe_layer_forward) run the same tile code and shapes: identical bits."""
    L = Layer(wl_of(*shape))
    try:
        a = L.forward().clone()
        out = torch.empty_like(a)
        moe.moe_expert_ffn(L.shape, L.x, L.ids, L.w, L.residency, out, L.ws)
        torch.cuda.synchronize()
        assert torch.equal(a, out)
    finally:
        L.close()


def test_single_token_repeated_calls_and_alternating_entry_points():
    """Back-to-back calls through either entry point on one workspace give the
    same bits every time (nothing carries over in the workspace)."""
    L = Layer(wl_of("f_rep", 1024, 512, 16, 4, 2))
    try:
        first = L.forward().clone()
        outs = []
        for i in range(6):
            if i % 2:
                o = torch.empty_like(first)
                moe.moe_expert_ffn(L.shape, L.x, L.ids, L.w, L.residency, o, L.ws)
                outs.append(o)
            else:
                outs.append(L.forward().clone())
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o, first)
    finally:
        L.close()


@pytest.mark.parametrize("T", [1, 2])
def test_single_token_cold_part_equals_all_hot_bitwise(T):
    """With cold experts picked, the hot experts' gate/up runs while the
    gather copies, then the cold experts' gate/up and the down + combine over
    all: the bits equal the all-resident launch, and the output matches the
    oracle."""
    wl = wl_of("f_cold", 1024, 512, 16, 4, T)
    hot_all = Layer(wl, all_hot=True)
    ids = hot_all.ids
    try:
        b = hot_all.forward().clone()
        torch.cuda.synchronize()
        picked = sorted(set(hot_all.ids.cpu().numpy().ravel().tolist()))
        # make half of the picked experts cold
        cold = set(picked[::2])
        hot = [e for e in range(wl.n_experts) if e not in cold]
        mixed = Layer(wl, hot=hot)
        try:
            a = mixed.forward()
            torch.cuda.synchronize()
            assert torch.equal(mixed.ids, ids)
            assert torch.equal(a, b), "hot/cold placement changed the output bits"
            check_out(a.cpu().numpy(), oracle_out(mixed)["out"])
        finally:
            mixed.close()
    finally:
        hot_all.close()


def test_single_token_invalid_ids_contribute_zero():
    L = Layer(wl_of("f_bad", 1024, 512, 16, 4, 2))
    try:
        L.forward()
        torch.cuda.synchronize()
        ids_g, w_g = L.ids.cpu().numpy(), L.w.cpu().numpy()
        bad = ids_g.copy()
        bad[0, 1] = -1
        bad[1, 3] = L.E
        out = torch.empty((L.T, L.H), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(L.shape, L.x, torch.from_numpy(bad).cuda(), torch.from_numpy(w_g).cuda(), L.residency,
                           out, L.ws)
        torch.cuda.synchronize()
        y = oracle_out(L)["y"].copy()
        y[0, 1] = 0
        y[1, 3] = 0
        check_out(out.cpu().numpy(), combine(w_g, y))
    finally:
        L.close()


def test_single_token_unusable_residency_entry_contributes_zero():
    L = Layer(wl_of("f_unusable", 1024, 512, 16, 4, 1))
    try:
        L.forward()
        torch.cuda.synchronize()
        ids_g, w_g = L.ids.cpu().numpy(), L.w.cpu().numpy()
        e_bad = int(ids_g[0, 2])
        slot = L.slot_np.copy()
        slot[e_bad] = L.n_hot + 3
        r = moe.residency(torch.from_numpy(slot).cuda(), L.hot_base, None, None, L.n_hot, 0)
        out = torch.empty((L.T, L.H), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(L.shape, L.x, L.ids, L.w, r, out, L.ws)
        torch.cuda.synchronize()
        y = oracle_out(L)["y"].copy()
        y[ids_g == e_bad] = 0
        check_out(out.cpu().numpy(), combine(w_g, y))
    finally:
        L.close()


def test_single_token_bf16_output_is_rounded_fp32():
    L = Layer(wl_of("f_bf16", 1024, 512, 16, 4, 2))
    try:
        f = L.forward().clone()
        b = L.forward(out_bf16=True)
        torch.cuda.synchronize()
        assert torch.equal(b, f.to(torch.bfloat16))
    finally:
        L.close()
