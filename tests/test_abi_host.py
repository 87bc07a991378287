"""The C-ABI library without a GPU: it loads, exports every entry point that
include/moe.h declares, and its host-only paths (sizes, shape and residency
validation, argument errors raised before any HIP call) behave as documented."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("moe_routed_expert_router_amd",
                          reason="libmoe.so not built (python moe_routed_expert_router_amd/build.py)")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(moe.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    assert moe.moe_status_string(0) == "MOE_OK"
    assert moe.moe_status_string(5) == "MOE_ERR_BAD_RESIDENCY"
    assert moe.moe_status_string(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("H,I,B", [(256, 128, 52224), (4096, 2048, 13369344)])
def test_expert_bytes(H, I, B):
    assert moe.moe_expert_bytes(moe.shape(H, I, 8, 2)) == B


def test_workspace_bytes():
    s = moe.shape(4096, 2048, 384, 6)
    w1, w8, w8192 = (moe.moe_workspace_bytes(s, t) for t in (1, 8, 8192))
    assert 0 < w1 < w8 < w8192
    assert w8192 >= 8192 * 6 * (4096 * 4 + 2048 * 4)     # per-pair y and h buffers
    assert moe.moe_workspace_bytes(s, -1) == 0
    assert moe.moe_workspace_bytes(moe.shape(100, 128, 8, 2), 1) == 0


@pytest.mark.parametrize("H,I,E,k,status", [
    (4096, 2048, 384, 6, moe.MOE_OK),
    (256, 128, 8, 2, moe.MOE_OK),
    (128, 128, 1024, 32, moe.MOE_OK),
    (100, 128, 8, 2, moe.MOE_ERR_UNSUPPORTED_SHAPE),
    (256, 96, 8, 2, moe.MOE_ERR_UNSUPPORTED_SHAPE),
    (256, 128, 1025, 2, moe.MOE_ERR_UNSUPPORTED_SHAPE),
    (256, 128, 8, 9, moe.MOE_ERR_UNSUPPORTED_SHAPE),
    (256, 128, 64, 33, moe.MOE_ERR_UNSUPPORTED_SHAPE),
    (256, 128, 8, 0, moe.MOE_ERR_INVALID_ARG),
    (0, 128, 8, 2, moe.MOE_ERR_INVALID_ARG),
])
def test_shape_check(H, I, E, k, status):
    assert moe.moe_shape_check(moe.shape(H, I, E, k)) == status


def test_residency_check():
    s = moe.shape(256, 128, 6, 2)
    moe.moe_residency_check(s, np.array([0, -1, 1, -2, -3, 2]), 3, 3)
    moe.moe_residency_check(s, np.arange(6), 6, 0)
    moe.moe_residency_check(s, -np.arange(6) - 1, 0, 6)
    bad = [
        (np.array([0, -1, 1, -2, -3, 2]), 4, 2),       # counts disagree with entries
        (np.array([0, -1, 0, -2, -3, 2]), 3, 3),       # hot index repeated
        (np.array([0, -1, 1, -1, -3, 2]), 3, 3),       # cold slot repeated
        (np.array([0, -1, 3, -2, -3, 2]), 3, 3),       # hot index out of range
        (np.array([0, -1, 1, -2, -4, 2]), 3, 3),       # cold slot out of range
        (np.arange(6), 5, 0),                           # n_hot + n_cold != E
    ]
    for slot, nh, nc in bad:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_residency_check(s, slot, nh, nc)
        assert ei.value.status == moe.MOE_ERR_BAD_RESIDENCY, (slot, nh, nc)


def test_null_arguments_rejected_before_any_launch():
    lib = moe.lib
    s = moe.shape(256, 128, 8, 2)
    st = lib.moe_route(ctypes.byref(s), 4, None, None, None, 1, None, None, None, None, 0, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "x is NULL" in moe.moe_last_error()
    bad = moe.shape(100, 128, 8, 2)
    st = lib.moe_route(ctypes.byref(bad), 4, None, None, None, 1, None, None, None, None, 0, None)
    assert st == moe.MOE_ERR_UNSUPPORTED_SHAPE
    st = lib.moe_route(ctypes.byref(s), -1, None, None, None, 1, None, None, None, None, 0, None)
    assert st == moe.MOE_ERR_UNSUPPORTED_SHAPE
    # zero tokens: nothing to do, nothing touched
    assert lib.moe_route(ctypes.byref(s), 0, None, None, None, 1, None, None, None, None, 0, None) == moe.MOE_OK
    r = moe.residency(None, None, None, None, 4, 3)
    st = lib.moe_layer_forward(ctypes.byref(s), 1, None, None, None, 1, ctypes.byref(r), None, None, 0, None,
                               None, 0, None)
    assert st == moe.MOE_ERR_BAD_RESIDENCY
    st = lib.moe_layer_forward(ctypes.byref(s), 1, None, None, None, 1, None, None, None, 0, None, None, 0, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = lib.moe_pick_set(ctypes.byref(s), 1, None, None, 9, 0, None, None, None, 0, None)
    assert st == moe.MOE_ERR_BAD_RESIDENCY
    with pytest.raises(moe.MoeError):
        moe.moe_host_free(0)


# ------------------------- adaptive residency (host) -------------------------
def _random_table(rng, E, n_hot):
    hot = set(rng.choice(E, n_hot, replace=False).tolist())
    slot = np.empty(E, dtype=np.int32)
    h = c = 0
    for e in range(E):
        if e in hot:
            slot[e], h = h, h + 1
        else:
            slot[e], c = -c - 1, c + 1
    return slot


def test_residency_plan_matches_oracle(rng):
    """The library's swap rule (host C++) against oracle.residency, bit for
    bit: pairs, the updated table and the float64 scores, over many ticks."""
    from oracle import residency as ores
    for E, n_hot in ((8, 5), (64, 40), (384, 255)):
        s = moe.shape(256, 128, E, 2)
        for threshold, decay, min_score, max_swaps in ((3.0, 0.9, 1.0, 8), (1.5, 0.5, 0.5, 64), (1.0, 1.0, 0.0, 3)):
            slot = _random_table(rng, E, n_hot)
            score = np.zeros(E)
            o_slot, o_score = slot.copy(), score.copy()
            for tick in range(12):
                # drifting skewed counts, with ties (integers) and quiet experts
                w = rng.permutation(E)[: max(1, E // 3)]
                counts = np.zeros(E, dtype=np.int32)
                counts[w] = rng.integers(0, 6, w.size)
                pairs = moe.moe_residency_plan(s, slot, n_hot, E - n_hot, score, counts, decay, threshold,
                                               min_score, max_swaps)
                o_pairs, o_slot, o_score = ores.manager_tick(o_slot, o_score, counts, decay, threshold, min_score,
                                                             max_swaps)
                assert [tuple(p) for p in pairs.tolist()] == o_pairs, (E, tick)
                assert np.array_equal(slot, o_slot)
                assert np.array_equal(score.view(np.uint64), o_score.view(np.uint64))
                moe.moe_residency_check(s, slot, n_hot, E - n_hot)


def test_residency_plan_rejects_bad_input():
    s = moe.shape(256, 128, 8, 2)
    slot = np.array([0, 1, 2, 3, 4, -1, -2, -3], dtype=np.int32)
    ok = dict(decay=0.5, threshold=3.0, min_score=1.0, max_swaps=4)
    cases = [
        (dict(ok, decay=1.5), "decay"), (dict(ok, threshold=0.0), "threshold"),
        (dict(ok, min_score=-1.0), "min_score"), (dict(ok, max_swaps=moe.MOE_MAX_SWAPS + 1), "max_swaps"),
    ]
    for kw, what in cases:
        score = np.zeros(8)
        before = slot.copy()
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_residency_plan(s, slot, 5, 3, score, np.zeros(8, np.int32), **kw)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG and what in moe.moe_last_error()
        assert np.array_equal(slot, before)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_residency_plan(s, slot, 5, 3, np.full(8, np.nan), np.zeros(8, np.int32), **ok)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_residency_plan(s, np.array([0, 0, 2, 3, 4, -1, -2, -3], np.int32), 5, 3, np.zeros(8),
                               np.zeros(8, np.int32), **ok)
    assert ei.value.status == moe.MOE_ERR_BAD_RESIDENCY


def test_residency_device_calls_validate_first():
    lib = moe.lib
    s = moe.shape(256, 128, 8, 2)
    r = moe.residency(None, None, None, None, 5, 3)
    pairs = (ctypes.c_int32 * 4)(5, 0, 6, 1)
    assert lib.moe_residency_swap(ctypes.byref(s), ctypes.byref(r), pairs, 65, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_residency_swap(ctypes.byref(s), ctypes.byref(r), pairs, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert "NULL" in moe.moe_last_error()
    bad = moe.residency(None, None, None, None, 5, 4)
    assert lib.moe_residency_swap(ctypes.byref(s), ctypes.byref(bad), pairs, 2, None) == moe.MOE_ERR_BAD_RESIDENCY
    assert lib.moe_fingerprint(ctypes.byref(s), ctypes.byref(r), None, -1, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_count_picks(ctypes.byref(s), 4, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_count_picks(ctypes.byref(s), -1, None, None, 0, None) == moe.MOE_ERR_UNSUPPORTED_SHAPE
