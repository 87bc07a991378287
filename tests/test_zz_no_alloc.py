"""moe_layer_forward_noalloc (the entry point for callers that cannot
allocate) against moe_layer_forward on the same inputs: two calls in a row,
the second with fewer tokens, must give the same ids, weights and output bits
(the static workspace keeps the first call's contents); a call larger than
the static workspace is refused with nothing written."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_routed_expert_router_amd as moe  # noqa: E402
from synth import gen  # noqa: E402
from tests.gpu_checks import check_out, oracle_out  # noqa: E402
from tests.gpu_setup import Layer  # noqa: E402


def _both(L, T):
    """The layer on its first T tokens through both entry points."""
    x = L.x[:T]
    ids_a, w_a = torch.empty((T, L.k), dtype=torch.int32, device="cuda"), torch.empty((T, L.k), device="cuda")
    ids_b, w_b = torch.full((T, L.k), -5, dtype=torch.int32, device="cuda"), torch.full((T, L.k), 9.0, device="cuda")
    out_a = torch.empty((T, L.H), dtype=torch.float32, device="cuda")
    out_b = torch.full((T, L.H), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(L.shape, T), dtype=torch.uint8, device="cuda")
    if L.scratch is not None:
        L.scratch.fill_(0x3C)
    moe.moe_layer_forward(L.shape, x, L.wr, L.bias, True, L.residency, ids_a, w_a, out_a, ws)
    torch.cuda.synchronize()
    if L.scratch is not None:
        L.scratch.fill_(0xC3)
    moe.moe_layer_forward_noalloc(L.shape, x, L.wr, L.bias, True, L.residency, ids_b, w_b, out_b)
    torch.cuda.synchronize()
    return (ids_a, w_a, out_a), (ids_b, w_b, out_b)


@pytest.mark.parametrize("name,Ts", [("hotcold8", (32, 8)), ("hotcold8", (8, 1)), ("decode1", (4, 1)),
                                     ("tiny", (40, 6))])
def test_noalloc_equals_layer_forward(name, Ts):
    """hotcold8 at 32 then 8 tokens: the existing entry point overlaps the
    gather on its side stream, the static one runs in order; 8 then 1 and the
    resident decode layer at 4 then 1: the one-token sequences; tiny at 40
    then 6: the many-token path, then a decode size."""
    wl = gen.workload(name)
    L = Layer(wl, T=max(Ts))
    try:
        for T in Ts:
            a, b = _both(L, T)
            assert torch.equal(a[0], b[0]), (name, T)
            assert torch.equal(a[1], b[1]), (name, T)
            assert torch.equal(a[2], b[2]), (name, T)
        ref = oracle_out(L, rows=[0])
        check_out(b[2].cpu().numpy()[:1], ref["out"])
    finally:
        L.close()


def test_noalloc_refuses_more_than_its_workspace():
    L = Layer(gen.workload("tiny"), T=8000)
    assert moe.moe_workspace_bytes(L.shape, L.T) > moe.MOE_NOALLOC_WS_BYTES
    L.ids.fill_(-3)
    L.out.fill_(5.0)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(L.shape, L.x, L.wr, L.bias, True, L.residency, L.ids, L.w, L.out)
    assert e.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(L.out == 5.0) and torch.all(L.ids == -3)
