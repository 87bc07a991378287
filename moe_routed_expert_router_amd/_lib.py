"""ctypes binding of libmoe.so: argument marshalling only.

Every function here has the name and argument order of the C entry point in
include/moe.h; tensors are passed as device pointers (torch is used only for
memory and streams).  A non-OK status raises MoeError with the library's own
error text.  There is no fallback: if libmoe.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int32, c_size_t, c_void_p, c_char_p, POINTER

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

# every entry point declared in include/moe.h
EXPORTS = (
    "moe_status_string", "moe_last_error", "moe_shape_check", "moe_expert_bytes",
    "moe_workspace_bytes", "moe_residency_check", "moe_host_alloc", "moe_host_free",
    "moe_route", "moe_pick_set", "moe_gather_cold", "moe_expert_ffn", "moe_layer_forward",
    "moe_count_picks", "moe_residency_plan", "moe_residency_swap", "moe_fingerprint",
    "moe_profile_enable", "moe_profile_reset", "moe_profile_read", "moe_probe_read", "moe_probe_mfma",
    "moe_layer_forward_noalloc",
)

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED_SHAPE = 2
MOE_ERR_MISALIGNED = 3
MOE_ERR_NOT_DEVICE_ACCESSIBLE = 4
MOE_ERR_BAD_RESIDENCY = 5
MOE_ERR_WORKSPACE_TOO_SMALL = 6
MOE_ERR_HIP = 7
MOE_OUT_F32, MOE_OUT_BF16 = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("inter", c_int32), ("n_experts", c_int32), ("top_k", c_int32)]


class MoeResidency(ctypes.Structure):
    _fields_ = [("slot", c_void_p), ("hot_base", c_void_p), ("host_cold", c_void_p),
                ("scratch", c_void_p), ("n_hot", c_int32), ("n_cold", c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python moe_routed_expert_router_amd/build.py")
    # One HIP runtime per process.  torch ships its own copy of the runtime
    # (same soname as the system one this library links); loaded first, it
    # also serves this library.  The other order would put two runtimes in the
    # process, and torch's device memory would be unknown to the library's.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "moe_status_string": (c_char_p, [c_int32]),
        "moe_last_error": (c_char_p, []),
        "moe_shape_check": (c_int32, [POINTER(MoeShape)]),
        "moe_expert_bytes": (c_size_t, [POINTER(MoeShape)]),
        "moe_workspace_bytes": (c_size_t, [POINTER(MoeShape), c_int32]),
        "moe_residency_check": (c_int32, [POINTER(MoeShape), P, c_int32, c_int32]),
        "moe_host_alloc": (c_int32, [c_size_t, c_int32, POINTER(c_void_p), POINTER(c_void_p)]),
        "moe_host_free": (c_int32, [P]),
        "moe_route": (c_int32, [POINTER(MoeShape), c_int32, P, P, P, c_int32, P, P, P, P, c_size_t, P]),
        "moe_pick_set": (c_int32, [POINTER(MoeShape), c_int32, P, P, c_int32, c_int32, P, P, P, c_size_t, P]),
        "moe_gather_cold": (c_int32, [POINTER(MoeShape), c_int32, P, POINTER(MoeResidency), P, c_size_t, P]),
        "moe_expert_ffn": (c_int32, [POINTER(MoeShape), c_int32, P, P, P, POINTER(MoeResidency), c_int32,
                                     P, P, c_size_t, P]),
        "moe_layer_forward": (c_int32, [POINTER(MoeShape), c_int32, P, P, P, c_int32,
                                        POINTER(MoeResidency), P, P, c_int32, P, P, c_size_t, P]),
        "moe_count_picks": (c_int32, [POINTER(MoeShape), c_int32, P, P, c_int32, P]),
        "moe_residency_plan": (c_int32, [POINTER(MoeShape), P, c_int32, c_int32, P, P, ctypes.c_double,
                                         ctypes.c_double, ctypes.c_double, c_int32, P, POINTER(c_int32)]),
        "moe_residency_swap": (c_int32, [POINTER(MoeShape), POINTER(MoeResidency), P, c_int32, P]),
        "moe_fingerprint": (c_int32, [POINTER(MoeShape), POINTER(MoeResidency), P, c_int32, P, P]),
        "moe_profile_enable": (c_int32, [c_int32]),
        "moe_profile_reset": (c_int32, []),
        "moe_profile_read": (c_int32, [c_int32, POINTER(c_char_p), POINTER(ctypes.c_int64),
                                       POINTER(ctypes.c_double)]),
        "moe_probe_read": (c_int32, [P, c_size_t, c_int32, P, P]),
        "moe_probe_mfma": (c_int32, [c_int32, c_int32, P, P]),
        "moe_layer_forward_noalloc": (c_int32, [POINTER(MoeShape), c_int32, P, P, P, c_int32,
                                                POINTER(MoeResidency), P, P, c_int32, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != MOE_OK:
        name = lib.moe_status_string(status).decode()
        raise MoeError(status, name, lib.moe_last_error().decode())


def _ptr(t) -> int | None:
    """Device (or mapped host) address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def shape(hidden: int, inter: int, n_experts: int, top_k: int) -> MoeShape:
    return MoeShape(hidden, inter, n_experts, top_k)


def residency(slot, hot_base, host_cold, scratch, n_hot: int, n_cold: int) -> MoeResidency:
    return MoeResidency(_ptr(slot), _ptr(hot_base), _ptr(host_cold), _ptr(scratch), n_hot, n_cold)


def _out_dtype(out) -> int:
    import torch
    if out.dtype == torch.float32:
        return MOE_OUT_F32
    if out.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MOE_OUT_BF16
    raise TypeError(f"out must be float32 or bf16, got {out.dtype}")


# ------------------------------- entry points -------------------------------
def moe_status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


def moe_shape_check(s: MoeShape) -> int:
    return lib.moe_shape_check(ctypes.byref(s))


def moe_expert_bytes(s: MoeShape) -> int:
    return lib.moe_expert_bytes(ctypes.byref(s))


def moe_workspace_bytes(s: MoeShape, n_tokens: int) -> int:
    return lib.moe_workspace_bytes(ctypes.byref(s), n_tokens)


def moe_residency_check(s: MoeShape, slot_host, n_hot: int, n_cold: int) -> None:
    """slot_host: a host int32 array (numpy) of E entries."""
    import numpy as np
    a = np.ascontiguousarray(slot_host, dtype=np.int32)
    _check(lib.moe_residency_check(ctypes.byref(s), a.ctypes.data, n_hot, n_cold))


def moe_host_alloc(nbytes: int, coherent: bool = False) -> tuple[int, int]:
    """(host address, device-visible address) of new pinned mapped host memory."""
    h, d = c_void_p(), c_void_p()
    _check(lib.moe_host_alloc(nbytes, 1 if coherent else 0, ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def moe_host_free(host_ptr: int) -> None:
    _check(lib.moe_host_free(host_ptr))


def moe_route(s: MoeShape, x, w_router, bias, renormalize: bool, topk_ids, topk_w, logits_out, ws,
              stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_route(ctypes.byref(s), T, _ptr(x), _ptr(w_router), _ptr(bias), int(bool(renormalize)),
                         _ptr(topk_ids), _ptr(topk_w), _ptr(logits_out), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)))


def moe_pick_set(s: MoeShape, topk_ids, slot, n_hot: int, n_cold: int, counts_out, cold_out, ws,
                 stream=None) -> None:
    T = topk_ids.shape[0]
    _check(lib.moe_pick_set(ctypes.byref(s), T, _ptr(topk_ids), _ptr(slot), n_hot, n_cold, _ptr(counts_out),
                            _ptr(cold_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_gather_cold(s: MoeShape, topk_ids, r: MoeResidency, ws, stream=None) -> None:
    T = topk_ids.shape[0]
    _check(lib.moe_gather_cold(ctypes.byref(s), T, _ptr(topk_ids), ctypes.byref(r), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_ffn(s: MoeShape, x, topk_ids, topk_w, r: MoeResidency, out, ws, stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_expert_ffn(ctypes.byref(s), T, _ptr(x), _ptr(topk_ids), _ptr(topk_w), ctypes.byref(r),
                              _out_dtype(out), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream)))


def moe_layer_forward(s: MoeShape, x, w_router, bias, renormalize: bool, r: MoeResidency, topk_ids, topk_w, out,
                      ws, stream=None) -> None:
    T = x.shape[0]
    _check(lib.moe_layer_forward(ctypes.byref(s), T, _ptr(x), _ptr(w_router), _ptr(bias), int(bool(renormalize)),
                                 ctypes.byref(r), _ptr(topk_ids), _ptr(topk_w), _out_dtype(out), _ptr(out),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


MOE_NOALLOC_WS_BYTES = 16 << 20


def moe_layer_forward_noalloc(s: MoeShape, x, w_router, bias, renormalize: bool, r: MoeResidency, topk_ids,
                              topk_w, out, stream=None) -> None:
    _check(lib.moe_layer_forward_noalloc(ctypes.byref(s), x.shape[0], _ptr(x), _ptr(w_router), _ptr(bias),
                                         1 if renormalize else 0, ctypes.byref(r), _ptr(topk_ids), _ptr(topk_w),
                                         _out_dtype(out), _ptr(out), _stream(stream)))


MOE_MAX_SWAPS = 64


def moe_count_picks(s: MoeShape, topk_ids, counts, clear: bool = False, stream=None) -> None:
    T = topk_ids.shape[0] if topk_ids is not None else 0
    _check(lib.moe_count_picks(ctypes.byref(s), T, _ptr(topk_ids), _ptr(counts), int(bool(clear)),
                               _stream(stream)))


def moe_residency_plan(s: MoeShape, slot_host, n_hot: int, n_cold: int, score, counts_host, decay: float,
                       threshold: float, min_score: float, max_swaps: int):
    """Host-only.  slot_host (int32) and score (float64) are numpy arrays
    updated in place; returns the pairs as an int32 array [n][2]."""
    import numpy as np
    for name, a, dt in (("slot_host", slot_host, np.int32), ("score", score, np.float64)):
        if not (isinstance(a, np.ndarray) and a.dtype == dt and a.flags.c_contiguous):
            raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dt).name} array (updated in place)")
    counts = np.ascontiguousarray(counts_host, dtype=np.int32)
    pairs = np.zeros((max(max_swaps, 1), 2), dtype=np.int32)
    n = c_int32()
    _check(lib.moe_residency_plan(ctypes.byref(s), slot_host.ctypes.data, n_hot, n_cold, score.ctypes.data,
                                  counts.ctypes.data, decay, threshold, min_score, max_swaps, pairs.ctypes.data,
                                  ctypes.byref(n)))
    return pairs[:n.value].copy()


def moe_residency_swap(s: MoeShape, r: MoeResidency, pairs, stream=None) -> None:
    """pairs: host int32 [n][2] (cold expert, hot expert)."""
    import numpy as np
    a = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    _check(lib.moe_residency_swap(ctypes.byref(s), ctypes.byref(r), a.ctypes.data if a.size else None,
                                  a.shape[0], _stream(stream)))


def moe_fingerprint(s: MoeShape, r: MoeResidency, experts, out, stream=None) -> None:
    _check(lib.moe_fingerprint(ctypes.byref(s), ctypes.byref(r), _ptr(experts), experts.numel(), _ptr(out),
                               _stream(stream)))


def moe_profile_enable(on: bool) -> None:
    _check(lib.moe_profile_enable(1 if on else 0))


def moe_profile_reset() -> None:
    _check(lib.moe_profile_reset())


def moe_profile_read() -> dict:
    """{kernel name: (launch count, total milliseconds)} of the recorded launches."""
    out = {}
    i = 0
    while True:
        name, cnt, ms = c_char_p(), ctypes.c_int64(), ctypes.c_double()
        if lib.moe_profile_read(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)) != MOE_OK:
            return out
        out[name.value.decode()] = (cnt.value, ms.value)
        i += 1


def moe_probe_read(src, nbytes: int, loads_per_thread: int, sink, stream=None) -> None:
    _check(lib.moe_probe_read(_ptr(src), nbytes, loads_per_thread, _ptr(sink), _stream(stream)))


def moe_probe_mfma(kind: int, iters: int, sink, stream=None) -> None:
    _check(lib.moe_probe_mfma(kind, iters, _ptr(sink), _stream(stream)))
