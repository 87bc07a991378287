"""Benchmark of the routed-expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole layer (router, pick set, cold gather when
experts are cold, grouped SwiGLU FFN, combine) over one batch of synthetic
tokens, through the C ABI.  The headline workload is one decode token through
one layer with all 384 MXFP4 experts resident (4096 hidden, 2048 expert width,
top-6).  Steps rotate over a pool of token batches so consecutive steps pick
different experts and the 256 MB Infinity Cache cannot serve repeated weight
bytes; the timed steps are replayed from a HIP graph captured over the pool.

Besides the one JSON line on stdout (rank 0), per-kernel durations come from
HIP events the library records around its own launches (moe_profile_*), in
a separate eager pass of the same steps, and the CPU oracle is timed on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-expert layer tokens/s + achieved HBM & host-link GB/s at batch 1/8/32"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0      # MI355X dense bf16 matrix cores, 2.5 PFLOP/s
DOWN_COMBINE_MAX_PAIRS = 8       # T*k up to which the library fuses the down projection and the combine
DOWN_BLOCKS_COMBINE_TOKENS = 16  # tokens below which the decode down blocks combine their row tiles themselves
LINK_PEAK_GBS = 64.0             # PCIe Gen5 x16, one direction
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed (string
    literals are kept; the sources put no comment markers inside them)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kernel: str, csrc: str | None = None) -> str:
    """Hash of the code (comments and layout ignored) of the source file that
    defines `kernel` plus every shared header: a counter summary stays valid
    while none of them changes."""
    import re
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "moe_routed_expert_router_amd", "csrc")
    files = sorted(os.listdir(csrc))
    pat = re.compile(r"__global__[^;{]*?\b" + re.escape(kernel) + r"\s*\(")
    for f in files:
        text = open(os.path.join(csrc, f), "rb").read().decode("utf-8", "replace")
        if f.endswith(".hpp") or (f.endswith(".hip") and pat.search(text)):
            h.update(f.encode())
            h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str) -> float | None:
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken from the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Workload:
    """Device inputs for `reps` batches of one workload, resident as it says."""

    def __init__(self, name: str, reps: int):
        import torch
        import moe_routed_expert_router_amd as moe
        from synth import gen
        from tests.gpu_setup import Layer
        self.wl = gen.workload(name)
        self.reps = reps
        self.Tb = self.wl.tokens
        self.layer = Layer(self.wl, T=self.Tb * reps)
        L = self.layer
        self.outs = [torch.empty((self.Tb, L.H), dtype=torch.float32, device="cuda") for _ in range(reps)]
        self.ids = [torch.empty((self.Tb, L.k), dtype=torch.int32, device="cuda") for _ in range(reps)]
        self.ws_ = [torch.empty((self.Tb, L.k), dtype=torch.float32, device="cuda") for _ in range(reps)]
        self.ws = torch.empty(moe.moe_workspace_bytes(L.shape, self.Tb), dtype=torch.uint8, device="cuda")

    def step(self, i: int, stream=None):
        import moe_routed_expert_router_amd as moe
        L = self.layer
        r = i % self.reps
        x = L.x[r * self.Tb:(r + 1) * self.Tb]
        moe.moe_layer_forward(L.shape, x, L.wr, L.bias, True, L.residency, self.ids[r], self.ws_[r],
                              self.outs[r], self.ws, stream)

    def picks(self):
        return np.concatenate([t.cpu().numpy() for t in self.ids])

    def close(self):
        self.layer.close()


REPEATS = 3          # timed repeats of the K steps; the figure is their median
AGREE = 0.02         # repeats agree when (max - min) / median is within 2%


def spread(xs) -> float:
    xs = sorted(xs)
    return (xs[-1] - xs[0]) / xs[len(xs) // 2]


def time_steps(w: Workload, steps: int, warmup: int, use_graph: bool, repeats: int = REPEATS):
    """Seconds of exactly `steps` whole-layer steps (step i runs batch i mod
    the pool size), timed `repeats` times after `warmup` untimed eager steps.
    With a graph, the K steps are captured once (one untimed replay) and each
    repeat is one replay.  Returns (list of seconds per repeat, graph used)."""
    import torch
    for i in range(warmup):
        w.step(i)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s, capture_error_mode="relaxed"):
                for i in range(steps):
                    w.step(i, stream=s)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported: time eagerly instead
            log(f"graph capture failed ({e}); timing eager launches")
            graph = None
            torch.cuda.synchronize()
    graphed = graph is not None
    secs = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                w.step(i)
        torch.cuda.synchronize()
        secs.append(time.perf_counter() - t0)
    del graph
    return secs, graphed


def profile_kernels(w: Workload, steps: int, repeats: int = REPEATS):
    """Per-kernel (launches per pass, median over `repeats` passes of the mean
    microseconds) from the library's HIP events, over eager passes of
    `steps` steps; and per kernel the spread of those means."""
    import torch
    import moe_routed_expert_router_amd as moe
    runs = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        moe.moe_profile_reset()
        moe.moe_profile_enable(True)
        for i in range(steps):
            w.step(i)
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        stats = moe.moe_profile_read()
        moe.moe_profile_reset()
        runs.append({k: (n, 1e3 * ms / n) for k, (n, ms) in stats.items() if n})
    prof, spreads = {}, {}
    for k in runs[0]:
        us = [r[k][1] for r in runs if k in r]
        prof[k] = (runs[0][k][0], float(np.median(us)))
        spreads[k] = spread(us)
    return prof, spreads


def ffn_bytes(w: Workload, picks_per_step: list[np.ndarray]) -> dict:
    """Algorithmic HBM bytes per launch, averaged over the steps' batches:
    each distinct picked expert's planes read once, activations read, results
    written (no re-reads counted)."""
    return layer_bytes([(w.layer, ids) for ids in picks_per_step])


def layer_bytes(layer_picks) -> dict:
    """As ffn_bytes, over (layer, ids of one launch) pairs (layers may differ).
    "combine": the separate combine kernel's y read and out write (0 where
    the down kernel combines itself)."""
    gu, dn, cb, cold_bytes, uniq = [], [], [], [], []
    for L, ids in layer_picks:
        H, I, k = L.H, L.I, L.k
        w13 = 2 * I * (H // 2) + 2 * I * (H // 32)
        w2 = H * (I // 2) + H * (I // 32)
        U = len(np.unique(ids))
        T = ids.shape[0]
        P = T * k
        gu.append(U * w13 + T * H * 2 + P * I * 4)           # + x read, h (hi+lo) write
        if P <= DOWN_COMBINE_MAX_PAIRS:                      # fused down + combine: + h read, out write
            dn.append(U * w2 + P * I * 4 + T * H * 4)
            cb.append(0)
        elif T < DOWN_BLOCKS_COMBINE_TOKENS:                 # + h read, y write, and the combine's y read, out write
            dn.append(U * w2 + P * I * 4 + P * H * 4 + P * H * 4 + T * H * 4)
            cb.append(0)
        else:                                                # + h read, y write; combine: y read, out write
            dn.append(U * w2 + P * I * 4 + P * H * 4)
            cb.append(P * H * 4 + T * H * 4)
        cold_bytes.append(sum(1 for e in np.unique(ids) if L.slot_np[e] < 0) * L.B)
        uniq.append(U)
    return {"gate_up": float(np.mean(gu)), "down": float(np.mean(dn)), "combine": float(np.mean(cb)),
            "gather_cold": float(np.mean(cold_bytes)), "unique": float(np.mean(uniq))}


def kernel_role(name: str) -> str | None:
    """Which algorithmic byte count a library kernel name is measured against."""
    if name.startswith("ffn_gate_up"):
        return "gate_up"
    if name.startswith("ffn_down"):
        return "down"
    if name == "gather_cold":
        return "gather_cold"
    if name == "ffn_combine":
        return "combine"
    return None


def forwards(prof: dict) -> int:
    """Layer forwards covered by a profile (every forward runs one router-logits kernel)."""
    return max(n for k, (n, _) in prof.items() if k.startswith("route_logits"))


def role_us(prof: dict, role: str) -> float:
    """Microseconds per layer forward spent in the kernels of one role (a role
    may run as several launches, e.g. the hot and the cold part of the FFN)."""
    per = forwards(prof)
    return sum(n * us for k, (n, us) in prof.items() if kernel_role(k) == role) / per


def kernel_table(prof: dict, by: dict) -> dict:
    """Per kernel: launches, mean duration and microseconds per layer forward;
    per FFN role: algorithmic bytes per forward over that role's time."""
    per = forwards(prof)
    out = {}
    for k, (n, us) in sorted(prof.items()):
        out[k] = {"launches": n, "mean_us": round(us, 3), "us_per_forward": round(n * us / per, 3)}
    for role in ("gate_up", "down", "combine", "gather_cold"):
        t = role_us(prof, role)
        if t > 0 and by.get(role):
            out[f"role:{role}"] = {"us_per_forward": round(t, 3), "algorithmic_bytes": int(by[role]),
                                   "GB_per_s": round(by[role] / (t * 1e-6) / 1e9, 1)}
    return out


def role_kernel(prof: dict, role: str) -> str:
    """The kernel of a role with the most time per forward."""
    return max((k for k in prof if kernel_role(k) == role), key=lambda k: prof[k][0] * prof[k][1])


def cpu_baseline(name: str, seconds: float) -> dict:
    """The oracle, untuned, on the host cores: one layer for one batch of the
    workload at a time, until about `seconds` of CPU work have run."""
    from synth import gen
    from oracle import layer as olayer
    blas = []
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads"), "version": i.get("version")}
                for i in info]
    except Exception:
        threads = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    wl = gen.workload(name)
    cal = gen.load_calibration() if wl.zipf else None
    bias = gen.zipf_prior(wl.seed, 0, wl.n_experts, cal["alpha"]) if wl.zipf else None
    wr = gen.router_weight(wl.seed, 0, wl.n_experts, wl.hidden)
    n_tok, elapsed, batches = 0, 0.0, 0
    max_batches = 64
    while elapsed < seconds and batches < max_batches:
        x = gen.tokens_bf16(wl.seed, 1000 + batches, wl.tokens, wl.hidden)
        # expert bytes are input generation: regenerate outside the timed region
        from oracle.route import route
        ids, _, _ = route(x, wr, bias, wl.top_k)
        blobs = {int(e): gen.expert_blob(wl.seed, 0, int(e), wl.hidden, wl.inter) for e in np.unique(ids)}
        t0 = time.perf_counter()
        olayer.layer_forward(x, wr, bias, lambda e: blobs[e], wl.hidden, wl.inter, wl.top_k)
        elapsed += time.perf_counter() - t0
        n_tok += wl.tokens
        batches += 1
    return {"value": n_tok / elapsed, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{batches} batches of {wl.tokens} token(s) of the {name} layer (seed {wl.seed}), "
                      f"{elapsed:.1f} s of oracle time (route, dequant, fp32 SwiGLU FFN, combine)",
            "host_cpus": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": cpu_model, "blas": blas}


def measure(name: str, steps: int, warmup: int, reps: int, use_graph: bool, prof_steps: int):
    """Timed steps (time_steps) and kernel profile (profile_kernels) of one
    workload; returns (workload, seconds per repeat, graph used, profile,
    profile spreads, algorithmic bytes)."""
    import torch
    w = Workload(name, min(reps, steps))
    try:
        secs, graphed = time_steps(w, steps, warmup, use_graph)
        # picks of the pool (the timed steps ran exactly these batches)
        torch.cuda.synchronize()
        picks = [t.cpu().numpy() for t in w.ids]
        prof, pspread = profile_kernels(w, prof_steps)
        by = ffn_bytes(w, picks)
        return w, secs, graphed, prof, pspread, by
    except Exception:
        w.close()
        raise


def layer_figures(name: str, steps: int, warmup: int, reps: int, use_graph: bool) -> dict:
    """Whole-layer figures of one workload: tokens/s (median of the timed
    repeats of exactly `steps` steps, with their spread), per-kernel times,
    the dominant kernel's roofline and the grouped FFN's HBM rate."""
    import torch
    w, secs, graphed, prof, pspread, by = measure(name, steps, warmup, reps, use_graph, min(steps, 256))
    try:
        wl = w.wl
        med = float(np.median(secs))
        rep = {"n": len(secs), "seconds": [round(x, 6) for x in secs], "spread": round(spread(secs), 4),
               "agree_within_2pct": spread(secs) <= AGREE}
        log(f"[bench] {name}: {steps} steps x {len(secs)} repeats, median {med:.4f} s "
            f"({1e6 * med / steps:.1f} us/step, spread {100 * spread(secs):.2f}%), graph={graphed}")
        kernels = kernel_table(prof, by)
        for k, e in kernels.items():
            if k in pspread:
                e["spread"] = round(pspread[k], 4)
            log(f"[bench]   {k:24s} {e['us_per_forward']:9.2f} us/forward" +
                (f"  {e['GB_per_s']:8.1f} GB/s" if "GB_per_s" in e else ""))
        dom = role_kernel(prof, "gate_up")
        dn = role_kernel(prof, "down")
        dom_us = prof[dom][1]
        achieved = by["gate_up"] / (dom_us * 1e-6) / 1e9
        ffn_us = role_us(prof, "gate_up") + role_us(prof, "down") + role_us(prof, "combine")
        ffn_gbs = (by["gate_up"] + by["down"] + by["combine"]) / (ffn_us * 1e-6) / 1e9
        if wl.tokens > 32:
            # prefill: the grouped GEMM is a dense contraction; its bound is
            # the bf16 matrix-core peak.  Algorithmic flops of gate/up: 2*P*H*2I.
            flops = 2.0 * wl.tokens * wl.top_k * wl.hidden * 2 * wl.inter
            tf = flops / (dom_us * 1e-6) / 1e12
            roofline = {"bound": "mfma", "kernel": dom, "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFS,
                        "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                        "flops_per_launch": flops, "mean_launch_us": round(dom_us, 3),
                        "spread": round(pspread[dom], 4), "hbm_GB_per_s": round(achieved, 1)}
            dflops = 2.0 * wl.tokens * wl.top_k * wl.inter * wl.hidden
            layer_flops = flops + dflops + 2.0 * wl.tokens * wl.n_experts * wl.hidden
            extra = {"down_kernel": dn, "down_TFLOP_per_s": round(dflops / (prof[dn][1] * 1e-6) / 1e12, 1),
                     "layer_useful_TFLOP_per_s": round(layer_flops * steps / med / 1e12, 1)}
        else:
            roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": read_traffic(dom, name), "bytes_per_launch": int(by["gate_up"]),
                        "mean_launch_us": round(dom_us, 3), "spread": round(pspread[dom], 4)}
            extra = {}
        out = {"tokens_per_s": round(steps * wl.tokens / med, 2), "ms_per_step": round(1e3 * med / steps, 5),
               "steps": steps, "repeats": rep, "graph": graphed, "mean_distinct_experts": round(by["unique"], 2),
               "roofline": roofline,
               "ffn": {"kernels": [dom, dn] + sorted(k for k in prof if kernel_role(k) == "combine"),
                       "us": round(ffn_us, 3), "hbm_GB_per_s": round(ffn_gbs, 1),
                       "frac": round(ffn_gbs / HBM_PEAK_GBS, 4)},
               "kernels": kernels, "_wl": wl}
        out.update(extra)
        if "gather_cold" in prof and by["gather_cold"] > 0:
            out["gather_link_GB_per_s"] = round(by["gather_cold"] / (role_us(prof, "gather_cold") * 1e-6) / 1e9, 2)
            out["gather_bytes_per_step"] = int(by["gather_cold"])
        return out
    finally:
        w.close()
        del w
        torch.cuda.empty_cache()


def measure_read_ceiling(sizes=(6291456, 26886144, 53534720, 80420864), launches: int = 24,
                         repeated=(6291456,)) -> dict:
    """The single-launch streaming-read ceiling: moe_probe_read over fresh
    bytes at each size (the decode1 router, down, gate/up and whole-FFN
    volumes), launches rotating over a pool larger than the Infinity Cache,
    kernel time from the library's launch events; the best of 1, 2, 4, 8 and
    16 loads per thread, with the median of the launches.  Sizes in
    `repeated` are measured again reading the same bytes every launch (as the
    router reads its weights every step), which the Infinity Cache can hold."""
    import torch
    import moe_routed_expert_router_amd as moe
    pool_bytes = max(1 << 30, 12 * max(sizes))
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    pool.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}

    def one(n16, rotate):
        slots = pool_bytes // n16 if rotate else 1
        best = None
        for lpt in (1, 2, 4, 8, 16):
            for i in range(4):   # untimed
                moe.moe_probe_read(pool[(i % slots) * n16:], n16, lpt, sink)
            torch.cuda.synchronize()
            us = []
            for i in range(launches):
                moe.moe_profile_reset()
                moe.moe_profile_enable(True)
                moe.moe_probe_read(pool[(i % slots) * n16:], n16, lpt, sink)
                torch.cuda.synchronize()
                moe.moe_profile_enable(False)
                cnt, ms = moe.moe_profile_read()["probe_read"]
                us.append(1e3 * ms / cnt)
            med = float(np.median(us))
            if best is None or med < best[1]:
                best = (lpt, med, spread(us))
        return best

    try:
        for n, rotate in [(n, True) for n in sizes] + [(n, False) for n in repeated]:
            n16 = n // 16 * 16
            lpt, med, sp = one(n16, rotate)
            gbs = n16 / (med * 1e-6) / 1e9
            key = f"{n16 / 1e6:.1f}MB" + ("" if rotate else "_repeated")
            out[key] = {"bytes": n16, "loads_per_thread": lpt, "kernel_us": round(med, 3),
                        "GB_per_s": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "spread": round(sp, 4)}
            log(f"[bench] read ceiling {n16 / 1e6:6.1f} MB{'' if rotate else ' (same bytes each launch)'}: "
                f"{med:7.2f} us = {gbs:7.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), {lpt} loads/thread")
        return out
    finally:
        moe.moe_profile_reset()
        del pool
        torch.cuda.empty_cache()


MFMA_KINDS = (   # (name, flops per instruction, published dense peak TFLOP/s or None)
    ("bf16 32x32x16", 32768, 2500.0),
    ("f8f6f4 32x32x64 fp8 x fp4", 131072, None),
    ("f8f6f4 32x32x64 fp8 x fp8", 131072, 5000.0),
    ("f8f6f4 32x32x64 fp6 x fp4", 131072, None),
    ("f8f6f4 32x32x64 fp4 x fp4", 131072, 10100.0),
)


def measure_mfma_rates(iters: int = 4096, launches: int = 5) -> dict:
    """Matrix-core rate of bf16 and of the scaled f8f6f4 forms with the GPU
    full (moe_probe_mfma: two 4-wave blocks per CU, four independent MFMAs
    per round), kernel time from the library's launch events, median of the
    launches.  The prefill gate/up would take x as a two-term fp8 split
    against fp4 weights: two fp8 x fp4 instructions per 32x32x64 step."""
    import torch
    import moe_routed_expert_router_amd as moe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    waves = 2 * cus * 4
    out = {}
    try:
        base = None
        for kind, (name, fpi, peak) in enumerate(MFMA_KINDS):
            for _ in range(2):   # untimed
                moe.moe_probe_mfma(kind, iters, sink)
            torch.cuda.synchronize()
            us = []
            for _ in range(launches):
                moe.moe_profile_reset()
                moe.moe_profile_enable(True)
                moe.moe_probe_mfma(kind, iters, sink)
                torch.cuda.synchronize()
                moe.moe_profile_enable(False)
                cnt, ms = moe.moe_profile_read()["probe_mfma"]
                us.append(1e3 * ms / cnt)
            med = float(np.median(us))
            tfs = waves * iters * 4 * fpi / (med * 1e-6) / 1e12
            base = base or tfs
            out[name] = {"kernel_us": round(med, 2), "TFLOP_per_s": round(tfs, 1), "vs_bf16": round(tfs / base, 3),
                         "frac_of_published_peak": round(tfs / peak, 3) if peak else None,
                         "spread": round(spread(us), 4)}
            log(f"[bench] mfma {name:28s}: {tfs:8.1f} TFLOP/s ({tfs / base:.2f}x bf16"
                + (f", {100 * tfs / peak:.0f}% of {peak / 1000:.1f} PFLOP/s" if peak else "") + ")")
        return out
    finally:
        moe.moe_profile_reset()


def measure_host_call(name: str = "decode1", calls: int = 200) -> dict:
    """Host time of one eager moe_layer_forward call (argument checks,
    pointer lookups and launches; the call does not wait for the GPU)."""
    import torch
    import moe_routed_expert_router_amd as moe
    from synth import gen
    from tests.gpu_setup import Layer
    L = Layer(gen.workload(name))
    try:
        for _ in range(10):
            L.forward()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream().cuda_stream
        t = []
        for i in range(calls):
            t0 = time.perf_counter()
            moe.moe_layer_forward(L.shape, L.x, L.wr, L.bias, True, L.residency, L.ids, L.w, L.out, L.ws, st)
            t.append(time.perf_counter() - t0)
            if i % 16 == 15:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        us = 1e6 * np.array(t)
        return {"workload": name, "calls": calls, "median_us": round(float(np.median(us)), 2),
                "p90_us": round(float(np.percentile(us, 90)), 2)}
    finally:
        L.close()


def measure_ffn_batches(batches=(1, 8, 32), layers: int = 4, reps: int = 10) -> dict:
    """The grouped FFN alone (moe_expert_ffn over every expert resident) at
    decode batch sizes, routed with the 40-layer workload's Zipf prior;
    `layers` independent layers rotate so that successive launches read
    different experts.  Kernel durations from the library's launch events."""
    import torch
    import moe_routed_expert_router_amd as moe
    from synth import gen
    from tests.gpu_setup import Layer
    wl = gen.workload("step40")
    out = {}
    for T in batches:
        Ls = [Layer(wl, layer=l, T=T, all_hot=True) for l in range(layers)]
        try:
            for L in Ls:
                L.forward()
            torch.cuda.synchronize()
            picks = [(L, L.ids.cpu().numpy()) for L in Ls]
            runs = []
            for it in range(1 + REPEATS):   # one untimed round, then the profiled ones
                if it:
                    moe.moe_profile_reset()
                    moe.moe_profile_enable(True)
                for _ in range(reps):
                    for L in Ls:
                        moe.moe_expert_ffn(L.shape, L.x, L.ids, L.w, L.residency, L.out, L.ws)
                torch.cuda.synchronize()
                if it:
                    moe.moe_profile_enable(False)
                    raw = moe.moe_profile_read()
                    moe.moe_profile_reset()
                    prof = {k: (n, 1e3 * ms / n) for k, (n, ms) in raw.items() if n}
                    per = layers * reps
                    runs.append({r: sum(n * u for k, (n, u) in prof.items() if kernel_role(k) == r) / per
                                 for r in ("gate_up", "down", "combine")})
            us = {r: float(np.median([x[r] for x in runs])) for r in ("gate_up", "down", "combine")}
            ffn_runs = [x["gate_up"] + x["down"] + x["combine"] for x in runs]
            by = layer_bytes(picks)
            ffn_us = us["gate_up"] + us["down"] + us["combine"]
            gbs = (by["gate_up"] + by["down"] + by["combine"]) / (ffn_us * 1e-6) / 1e9
            out[f"batch{T}"] = {
                "tokens": T, "mean_distinct_experts": round(by["unique"], 2),
                "gate_up_us": round(us["gate_up"], 3), "down_us": round(us["down"], 3),
                "combine_us": round(us["combine"], 3),
                "gate_up_GB_per_s": round(by["gate_up"] / (us["gate_up"] * 1e-6) / 1e9, 1),
                "down_GB_per_s": round(by["down"] / (us["down"] * 1e-6) / 1e9, 1),
                "ffn_hbm_GB_per_s": round(gbs, 1), "ffn_frac": round(gbs / HBM_PEAK_GBS, 4),
                "ffn_us_spread": round(spread(ffn_runs), 4)}
            log(f"[bench] ffn batch {T}: {ffn_us:.1f} us, {gbs:.0f} GB/s")
        finally:
            for L in Ls:
                L.close()
            del Ls
            torch.cuda.empty_cache()
    return out


def graph_us_per_layer(Ls, reps: int) -> float:
    """Mean microseconds per layer forward of the layers Ls run in order,
    captured once in a HIP graph and replayed `reps` times (event-timed, no
    host launch overhead)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for L in Ls:
            L.forward(stream=s.cuda_stream)
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s, capture_error_mode="relaxed"):
        for L in Ls:
            L.forward(stream=s.cuda_stream)
    graph.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    del graph
    return t0.elapsed_time(t1) * 1e3 / (reps * len(Ls))


def measure_verify(streams=(1, 2, 4, 8, 16), layers: int = 4, reps: int = 8) -> dict:
    """Speculative-verify decode steps on hot/cold layers (255 resident, 129
    gathered): S streams x (1 + draft) tokens, draft 5 at 1-4 streams and 1
    at 5-16, windows correlated so that a 1 + 5 window touches ~3.7x one
    token's experts.  Per S: us per layer forward (graph replay, `layers`
    layers rotating, each with its own cold pool), verified tokens/s per
    layer, distinct experts per window and per forward, cold bytes gathered
    per forward."""
    import torch
    from synth import gen
    from tests.gpu_setup import HostBuffer, Layer, fill_host_experts
    wl = gen.workload("hotcold8")
    cal = gen.load_calibration()
    rho = gen.load_verify_calibration()["rho"]
    B = gen.expert_bytes(wl.hidden, wl.inter)
    out = {}
    pools = []
    try:
        for l in range(layers):   # each layer's cold pool, shared by every stream count
            hot = set(gen.hot_set(wl.seed, l, cal))
            cold = [e for e in range(wl.n_experts) if e not in hot]
            pools.append(HostBuffer(len(cold) * B))
            fill_host_experts(pools[-1], wl.seed, l, cold, wl.hidden, wl.inter)
        for S in streams:
            out[f"streams{S}"] = _verify_point(wl, cal, rho, pools, S, reps)
    finally:
        for p in pools:
            p.close()
    return out


def _verify_point(wl, cal, rho, pools, S, reps):
    """One stream count of measure_verify (layers borrow the cold pools)."""
    import torch
    from synth import gen
    from tests.gpu_setup import Layer
    W = gen.verify_window(S)
    Ls = []
    try:
        for l, pool in enumerate(pools):
            x = gen.verify_tokens_bf16(wl.seed + 100, l, S, W, wl.hidden, rho)
            Ls.append(Layer(wl, layer=l, cal=cal, x_np=x, host=pool))
        us = graph_us_per_layer(Ls, reps)
        ids = [L.ids.cpu().numpy() for L in Ls]
        win = float(np.mean([len(np.unique(i[s * W:(s + 1) * W])) for i in ids for s in range(S)]))
        fwd = float(np.mean([len(np.unique(i)) for i in ids]))
        cold = float(np.mean([sum(1 for e in np.unique(i) if L.slot_np[e] < 0) * L.B
                              for i, L in zip(ids, Ls)]))
        T = S * W
        log(f"[bench] verify {S} streams x {W}: {us:.1f} us/layer, {win:.1f} experts per window "
            f"({win / wl.top_k:.2f}x one token), {cold / 1e6:.1f} MB cold per forward")
        return {"tokens": T, "window": W, "us_per_layer": round(us, 2),
                "verified_tokens_per_s_per_layer": round(T / (us * 1e-6), 1),
                "distinct_experts_per_window": round(win, 2),
                "window_over_one_token": round(win / wl.top_k, 3),
                "distinct_experts_per_forward": round(fwd, 2), "cold_bytes_per_forward": int(cold)}
    finally:
        for L in Ls:
            L.close()
        del Ls
        torch.cuda.empty_cache()


def measure_adaptive(layers: int = 8, warm: int = 1500, steps: int = 1000, drift: float = 0.2,
                     decay: float = 0.999, min_score: float = 1.0, max_swaps: int = 4,
                     thresholds=(None, 1.5, 3.0), pool: int = 1024, drift_every: int | None = None) -> dict:
    """Adaptive residency on drifting traffic: `layers` hot/cold decode layers
    (255 resident / 129 in pinned host memory, one stream, one token per
    step) whose traffic has drifted from the calibration the hot sets were
    chosen on (one round of drift over `drift` of the Zipf ranks).  Per mode
    (static map, or the manager with each hysteresis threshold): `warm`
    steps to adapt, then `steps` measured.  A step is the layers' forwards
    and pick counts replayed from one HIP graph; the manager reads the
    counts, plans on the host and enqueues the swaps between steps.  Reports
    forward and swap time per step, cold experts gathered and swaps per
    1000 steps, and a final byte audit of every expert against its boot
    fingerprint.  drift_every: the traffic keeps drifting, one more round
    every that many steps (mixed traffic that never settles)."""
    import torch
    import moe_routed_expert_router_amd as moe
    from synth import gen
    from tests.gpu_setup import Layer
    wl = gen.workload("hotcold8")
    cal = gen.load_calibration()
    E, H = wl.n_experts, wl.hidden
    Ls = []
    try:
        for l in range(layers):
            L = Layer(wl, layer=l, T=1, cal=cal)
            b = gen.drifted_zipf_prior(wl.seed, l, E, cal["alpha"], drift, 1)
            L.bias_np = b
            L.bias.copy_(torch.from_numpy(b))
            Ls.append(L)
        base_hot = [set(L.hot) for L in Ls]
        n_rounds = 1 + (0 if not drift_every else (warm + steps - 1) // drift_every)
        priors = [[torch.from_numpy(gen.drifted_zipf_prior(wl.seed, l, E, cal["alpha"], drift, r + 1)).cuda()
                   for r in range(n_rounds)] for l in range(layers)]
        toks = [torch.from_numpy(gen.tokens_bf16(wl.seed + 7, l, pool, H).view(np.int16)).cuda()
                for l in range(layers)]
        xbuf = [torch.empty((1, H), dtype=torch.int16, device="cuda") for _ in range(layers)]
        counts = torch.zeros((layers, E), dtype=torch.int32, device="cuda")
        all_e = torch.arange(E, dtype=torch.int32, device="cuda")
        fps = torch.empty((layers, E), dtype=torch.int64, device="cuda")

        def fingerprint_all():
            for l, L in enumerate(Ls):
                moe.moe_fingerprint(L.shape, L.residency, all_e, fps[l])
            torch.cuda.synchronize()
            return fps.cpu().numpy().copy()

        boot = fingerprint_all()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        for l, L in enumerate(Ls):
            L.x = xbuf[l]
            xbuf[l].copy_(toks[l][0:1])

        def body():
            for l, L in enumerate(Ls):
                L.forward(stream=s.cuda_stream)
                moe.moe_count_picks(L.shape, L.ids, counts[l], clear=True, stream=s.cuda_stream)

        with torch.cuda.stream(s):
            body()
        s.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s, capture_error_mode="relaxed"):
            body()
        torch.cuda.synchronize()

        def restore_map():
            # move the hot sets back to the calibrated ones (which slot holds
            # which expert does not matter)
            for l, L in enumerate(Ls):
                back_in = [e for e in base_hot[l] if L.slot_np[e] < 0]
                back_out = [e for e in range(E) if L.slot_np[e] >= 0 and e not in base_hot[l]]
                pairs = list(zip(back_in, back_out))
                for i in range(0, len(pairs), moe.MOE_MAX_SWAPS):
                    chunk = pairs[i:i + moe.MOE_MAX_SWAPS]
                    moe.moe_residency_swap(L.shape, L.residency, chunk)
                    for c, h in chunk:
                        L.slot_np[c], L.slot_np[h] = L.slot_np[h], L.slot_np[c]
            torch.cuda.synchronize()
            for L in Ls:
                assert np.array_equal(L.slot.cpu().numpy(), L.slot_np)

        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        out = {}
        for th in thresholds:
            name = "static" if th is None else f"adaptive_threshold{th:g}"
            restore_map()
            scores = [np.zeros(E) for _ in Ls]
            fwd_ms = swap_ms = 0.0
            cold_picks = swaps = 0
            t_host = 0.0
            for i in range(warm + steps):
                if i == 0 or (drift_every and i % drift_every == 0):
                    r = 0 if not drift_every else i // drift_every
                    for l, L in enumerate(Ls):
                        L.bias.copy_(priors[l][r])
                for l in range(layers):
                    xbuf[l].copy_(toks[l][i % pool:i % pool + 1])
                ev[0].record()
                graph.replay()                    # on the current stream, as everything below
                ev[1].record()
                c = counts.cpu().numpy()          # waits for the step
                measured = i >= warm
                if measured:
                    fwd_ms += ev[0].elapsed_time(ev[1])
                    cold_picks += sum(int(np.sum((c[l] > 0) & (L.slot_np < 0))) for l, L in enumerate(Ls))
                if th is None:
                    continue
                th0 = time.perf_counter()
                plans = [moe.moe_residency_plan(L.shape, L.slot_np, L.n_hot, L.n_cold, scores[l], c[l], decay,
                                                th, min_score, max_swaps) for l, L in enumerate(Ls)]
                t1 = time.perf_counter()
                n = sum(len(p) for p in plans)
                if n:
                    ev[2].record()
                    for L, p in zip(Ls, plans):
                        if len(p):
                            moe.moe_residency_swap(L.shape, L.residency, p)
                    ev[3].record()
                    if measured:
                        ev[3].synchronize()
                        swap_ms += ev[2].elapsed_time(ev[3])
                if measured:
                    swaps += n
                    t_host += t1 - th0
            torch.cuda.synchronize()
            B = Ls[0].B
            entry = {"forward_ms_per_step": round(fwd_ms / steps, 4),
                     "swap_ms_per_step": round(swap_ms / steps, 4),
                     "ms_per_step": round((fwd_ms + swap_ms) / steps, 4),
                     "tokens_per_s": round(steps / ((fwd_ms + swap_ms) * 1e-3), 1),
                     "cold_experts_per_step": round(cold_picks / steps, 3),
                     "gathered_MB_per_step": round(cold_picks * B / steps / 1e6, 2),
                     "swaps_per_1000_steps": round(1000 * swaps / steps, 1),
                     "moved_MB_per_step": round(2 * swaps * B / steps / 1e6, 2),
                     "plan_us_per_step": round(1e6 * t_host / steps, 1)}
            out[name] = entry
            log(f"[bench] residency {name}: forward {entry['forward_ms_per_step']:.3f} ms + swaps "
                f"{entry['swap_ms_per_step']:.3f} ms per step ({layers} layers, 1 token), "
                f"{entry['cold_experts_per_step']:.2f} cold experts/step, {entry['swaps_per_1000_steps']:.0f} "
                f"swaps per 1000 steps")
        after = fingerprint_all()
        mism = 0
        for l, L in enumerate(Ls):
            mism += int(np.sum(after[l] != boot[l]))
        out["audit"] = {"experts_checked": int(layers * E), "mismatches": mism}
        out["setup"] = {"layers": layers, "tokens_per_step": 1, "warm_steps": warm, "measured_steps": steps,
                        "drift_fraction": drift, "drift_every_steps": drift_every, "decay": decay,
                        "min_score": min_score,
                        "max_swaps_per_layer_tick": max_swaps}
        log(f"[bench] residency audit: {mism} mismatches over {layers * E} experts")
        del graph
        return out
    finally:
        for L in Ls:
            L.close()
        del Ls
        torch.cuda.empty_cache()


def measure_direct_read(batches=(1, 8, 32), layers: int = 4, reps: int = 8) -> dict:
    """Gather-then-compute against direct read (the FFN reads the picked cold
    experts in place from pinned host memory) for hot/cold decode layers
    (255 hot / 129 cold, Zipf routing) at each batch size: the whole layer
    per forward, `layers` layers rotating (each with its own cold pool, so
    no forward finds its host bytes in a GPU cache), replayed from a HIP
    graph per mode, event-timed."""
    import torch
    from synth import gen
    from tests.gpu_setup import Layer
    wl = gen.workload("hotcold8")
    cal = gen.load_calibration()
    out = {}
    for T in batches:
        G, D = [], []
        try:
            for l in range(layers):
                G.append(Layer(wl, layer=l, T=T, cal=cal))
                D.append(Layer(wl, layer=l, T=T, cal=cal, host=G[-1].host, direct=True))
            us = {name: graph_us_per_layer(Ls, reps) for name, Ls in (("gather", G), ("direct", D))}
            cold = float(np.mean([sum(1 for e in np.unique(L.ids.cpu().numpy()) if L.slot_np[e] < 0) * L.B
                                  for L in D]))
            out[f"batch{T}"] = {
                "tokens": T, "cold_bytes_per_forward": int(cold),
                "gather_us": round(us["gather"], 2), "direct_us": round(us["direct"], 2),
                "gather_tokens_per_s": round(T / (us["gather"] * 1e-6), 1),
                "direct_tokens_per_s": round(T / (us["direct"] * 1e-6), 1),
                "direct_over_gather": round(us["gather"] / us["direct"], 3)}
            log(f"[bench] direct read batch {T}: gather {us['gather']:.1f} us, direct {us['direct']:.1f} us, "
                f"{cold / 1e6:.1f} MB cold per forward")
        finally:
            for L in D + G:
                L.close()
            del G, D
            torch.cuda.empty_cache()
    return out


def pcie_link() -> dict:
    """Negotiated PCIe speed and width of GPU 0, from sysfs (empty when not
    readable)."""
    import torch
    try:
        pr = torch.cuda.get_device_properties(0)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        base = f"/sys/bus/pci/devices/{bdf}"
        out = {"bdf": bdf}
        for f in ("current_link_speed", "current_link_width", "max_link_speed", "max_link_width"):
            with open(os.path.join(base, f)) as fh:
                out[f] = fh.read().strip()
        return out
    except Exception as e:   # noqa: BLE001 - informational only
        return {"unavailable": f"{type(e).__name__}: {e}"}


def measure_gather_sweep(ms=(1, 2, 4, 8, 16, 64, 129), reps: int = 5) -> dict:
    """The cold gather alone with exactly m distinct cold experts picked
    (ids padded with hot experts), on a hot/cold decode layer: link GB/s =
    m * B / kernel time, beside the DMA engines copying the same bytes from
    pinned host memory (the practical ceiling) and the PCIe link's
    negotiated speed and width."""
    import torch
    import moe_routed_expert_router_amd as moe
    from synth import gen
    from tests.gpu_setup import Layer
    wl = gen.workload("hotcold8")
    k = wl.top_k
    L = Layer(wl, T=max(-(-m // k) for m in ms))
    out = {"link": pcie_link(), "peak_GB_per_s": LINK_PEAK_GBS}
    src = torch.empty(max(ms) * L.B, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty_like(src, device="cuda")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    try:
        for m in ms:
            T = -(-m // k)
            pad = L.cold[:m] + [L.hot[0]] * (T * k - m)
            ids = torch.tensor(pad, dtype=torch.int32, device="cuda").reshape(T, k)
            ws = torch.empty(moe.moe_workspace_bytes(L.shape, T), dtype=torch.uint8, device="cuda")
            ms_k = timed(lambda: moe.moe_gather_cold(L.shape, ids, L.residency, ws))
            n = m * L.B
            ms_d = timed(lambda: dst[:n].copy_(src[:n], non_blocking=True))
            out[f"m{m}"] = {"bytes": n, "kernel_us": round(1e3 * ms_k, 1),
                            "kernel_GB_per_s": round(n / ms_k / 1e6, 2),
                            "dma_GB_per_s": round(n / ms_d / 1e6, 2),
                            "frac_of_link": round(n / ms_k / 1e6 / LINK_PEAK_GBS, 3)}
            log(f"[bench] gather m={m:3d}: {1e3 * ms_k:9.1f} us, {n / ms_k / 1e6:5.1f} GB/s "
                f"(DMA {n / ms_d / 1e6:5.1f} GB/s)")
        return out
    finally:
        L.close()
        del src, dst
        torch.cuda.empty_cache()


def measure_layer_copy(T: int = 32, layers: int = 40, reps: int = 3) -> dict:
    """Layer-granular copy baseline: the layer's whole expert set (all 384
    experts, 5.13 GB, kept in pinned host memory as a layer offloader keeps
    it) copied to HBM before the layer runs, then the layer computed on the
    copy.  The copy is timed two ways: the gather kernel with every expert
    picked, and the DMA engines (the host pool copied into the same HBM area
    by hipMemcpyAsync); after each, all 384 copied blobs are compared with
    the host bytes.  The forward then runs with the copy as the layer's HBM
    pool and its output is compared with the same layer fully resident.  Per-
    step tokens/s is for `layers` such layers at T tokens each, to set
    beside the picked-only step of the same shape."""
    import torch
    import moe_routed_expert_router_amd as moe
    from synth import gen
    from tests.gpu_setup import Layer
    wl = gen.workload("hotcold8")
    E, k = wl.n_experts, wl.top_k
    L = Layer(wl, T=T, hot=[])        # nothing resident: the layer lives on the host
    try:
        B = L.B
        nbytes = E * B
        Tc = -(-E // k)
        pad = list(range(E)) + [0] * (Tc * k - E)
        ids = torch.tensor(pad, dtype=torch.int32, device="cuda").reshape(Tc, k)
        ws = torch.empty(moe.moe_workspace_bytes(L.shape, Tc), dtype=torch.uint8, device="cuda")
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            t0.record()
            for _ in range(reps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / reps

        host_dev = torch.from_numpy(L.host.np).cuda()   # the host bytes, for the comparisons
        dst = L.scratch.view(-1)
        dst.fill_(0)
        kern_ms = timed(lambda: moe.moe_gather_cold(L.shape, ids, L.residency, ws))
        gather_exact = bool(torch.equal(dst, host_dev))
        src = torch.from_numpy(L.host.np)              # the pinned pool itself
        assert src.is_pinned()
        dst.fill_(0)
        dma_ms = timed(lambda: dst.copy_(src, non_blocking=True))
        dma_exact = bool(torch.equal(dst, host_dev))
        del host_dev
        # the layer on its copy: expert e sits in row e of the copied area
        slot = torch.arange(E, dtype=torch.int32, device="cuda")
        r = moe.residency(slot, L.scratch, None, None, E, 0)
        out = torch.empty_like(L.out)

        def fwd():
            moe.moe_layer_forward(L.shape, L.x, L.wr, L.bias, True, r, L.ids, L.w, out, L.ws)

        fwd_ms = timed(fwd)
        ref = Layer(wl, T=T, all_hot=True)
        try:
            b = ref.forward()
            torch.cuda.synchronize()
            same_out = bool(torch.equal(out, b)) and bool(torch.equal(L.ids, ref.ids))
        finally:
            ref.close()
        copy_ms = min(kern_ms, dma_ms)
        step_ms = layers * (copy_ms + fwd_ms)
        res = {"bytes_per_layer": nbytes, "experts": E,
               "gather_kernel_ms": round(kern_ms, 3), "gather_kernel_GB_per_s": round(nbytes / kern_ms / 1e6, 2),
               "dma_copy_ms": round(dma_ms, 3), "dma_copy_GB_per_s": round(nbytes / dma_ms / 1e6, 2),
               "forward_on_copy_ms": round(fwd_ms, 4), "tokens_per_layer": T, "layers": layers,
               "ms_per_step": round(step_ms, 2), "tokens_per_s": round(T / (step_ms * 1e-3), 2),
               "gather_copy_bit_exact": gather_exact, "dma_copy_bit_exact": dma_exact,
               "blobs_compared": E, "forward_on_copy_equals_resident": same_out}
        log(f"[bench] layer copy: {nbytes / 1e9:.2f} GB per layer, kernel {kern_ms:.1f} ms "
            f"({nbytes / kern_ms / 1e6:.1f} GB/s), DMA {dma_ms:.1f} ms ({nbytes / dma_ms / 1e6:.1f} GB/s); "
            f"forward on the copy {fwd_ms:.3f} ms (= resident: {same_out}); "
            f"{layers} layers x {T} tokens: {res['tokens_per_s']} tok/s")
        return res
    finally:
        L.close()
        del L
        torch.cuda.empty_cache()


def _stack_batch1(S, rows: int, steps: int) -> dict:
    """One-stream decode steps on the same resident stack: one token per
    layer, the token taken from row r of each layer's batch for step r (mod
    rows), each row's 40-layer pass replayed from its own HIP graph; the
    cold experts each step gathers are counted from the routing, and one
    profiled eager pass over every row gives the gather's share of the
    kernel time."""
    import torch
    import moe_routed_expert_router_amd as moe
    full = [(L.x, L.ids, L.w, L.out) for L in S.layers]
    ids_full = [L.ids.cpu().numpy() for L in S.layers]

    def use_row(r):
        for L, (x, ids, w, out) in zip(S.layers, full):
            L.x, L.ids, L.w, L.out = x[r:r + 1], ids[r:r + 1], w[r:r + 1], out[r:r + 1]

    graphs = []
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        for r in range(rows):
            use_row(r)
            S.forward()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
                S.forward(stream=s)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % rows].replay()
        torch.cuda.synchronize()
        secs = time.perf_counter() - t0
        moe.moe_profile_reset()
        moe.moe_profile_enable(True)
        for r in range(rows):
            use_row(r)
            S.forward()
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        stats = moe.moe_profile_read()
        moe.moe_profile_reset()
    finally:
        del graphs
        for L, (x, ids, w, out) in zip(S.layers, full):
            L.x, L.ids, L.w, L.out = x, ids, w, out
    total_ms = sum(ms for _, ms in stats.values())
    gather_ms = stats.get("gather_cold", (0, 0.0))[1]
    cold = [sum(1 for e in set(ids_full[l][r].tolist()) if L.slot_np[e] < 0) for r in range(rows)
            for l, L in enumerate(S.layers)]
    res = {"tokens_per_s": round(steps / secs, 1), "ms_per_step": round(1e3 * secs / steps, 4),
           "token_rows_rotated": rows, "cold_experts_per_step": round(sum(cold) / rows, 2),
           "gather_ms_per_step": round(gather_ms / rows, 4),
           "gather_share_of_kernel_time": round(gather_ms / total_ms, 3) if total_ms else None}
    log(f"[bench] one stream: {res['ms_per_step']:.3f} ms/step ({res['tokens_per_s']} tokens/s), "
        f"{res['cold_experts_per_step']} cold experts gathered per step, gather "
        f"{res['gather_ms_per_step']:.3f} ms/step")
    return res


def measure_stack(name: str, steps: int, warmup: int, use_graph: bool, one_token_rows: int = 0,
                  steps_batch1: int = 64) -> dict:
    """Whole decode steps of a multi-layer workload (every layer in order on
    one stream, one shared cold scratch); None if it does not fit the GPU.
    one_token_rows > 0 adds one-stream steps (one token per layer) on the
    same stack."""
    import torch
    import moe_routed_expert_router_amd as moe
    from synth import gen
    from tests.gpu_setup import Stack
    wl = gen.workload(name)
    B = gen.expert_bytes(wl.hidden, wl.inter)
    need = (wl.layers * wl.hot_count + wl.n_cold) * B
    free = torch.cuda.mem_get_info()[0]
    if free < need * 1.05:
        log(f"[bench] {name}: needs {need / 2**30:.1f} GiB of device memory, {free / 2**30:.1f} free; skipped")
        return {"skipped": f"needs {need / 2**30:.1f} GiB of device memory, {free / 2**30:.1f} GiB free"}
    t0 = time.perf_counter()
    # pinned host memory is capped near 66 GiB on these hosts and the 40 cold pools
    # need 64.25 GiB: keep headroom, later layers reuse earlier pools
    S = Stack(wl, log=log, share_host_on_oom=True, max_host_pools=36)
    log(f"[bench] {name}: {wl.layers} layers resident in {time.perf_counter() - t0:.1f} s")
    try:
        for _ in range(warmup):
            S.forward()
        torch.cuda.synchronize()
        graph = None
        if use_graph:
            try:
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=s, capture_error_mode="relaxed"):
                    S.forward(stream=s)
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
            except Exception as e:
                log(f"[bench] {name}: graph capture failed ({e}); timing eager steps")
                graph = None
        reps = []
        for _ in range(REPEATS):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                if graph is not None:
                    graph.replay()
                else:
                    S.forward()
            torch.cuda.synchronize()
            reps.append(time.perf_counter() - t0)
        secs = float(np.median(reps))
        picks = [(L, L.ids.cpu().numpy()) for L in S.layers]
        moe.moe_profile_reset()
        moe.moe_profile_enable(True)
        S.forward()
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        stats = moe.moe_profile_read()
        moe.moe_profile_reset()
        prof = {k: (n, 1e3 * ms / n) for k, (n, ms) in stats.items() if n}
        by = layer_bytes(picks)
        kt = kernel_table(prof, by)
        ffn_us = role_us(prof, "gate_up") + role_us(prof, "down") + role_us(prof, "combine")
        entry = {"tokens_per_s": round(steps * wl.tokens / secs, 2), "ms_per_step": round(1e3 * secs / steps, 4),
                 "layers": wl.layers, "tokens_per_layer": wl.tokens, "steps": steps, "graph": graph is not None,
                 "repeats": {"n": len(reps), "seconds": [round(x, 5) for x in reps], "spread": round(spread(reps), 4),
                             "agree_within_2pct": spread(reps) <= AGREE},
                 "distinct_cold_pools": S.distinct_host_pools,
                 "mean_distinct_experts_per_layer": round(by["unique"], 2),
                 "ffn_hbm_GB_per_s": round((by["gate_up"] + by["down"] + by["combine"]) / (ffn_us * 1e-6) / 1e9, 1),
                 "kernels_per_layer": kt}
        if "gather_cold" in prof and by["gather_cold"] > 0:
            entry["gather_link_GB_per_s"] = round(by["gather_cold"] / (role_us(prof, "gather_cold") * 1e-6) / 1e9, 2)
            entry["gather_bytes_per_layer"] = int(by["gather_cold"])
        log(f"[bench] {name}: {entry['ms_per_step']:.3f} ms/step, {entry['tokens_per_s']} tokens/s")
        if one_token_rows:
            entry["batch1"] = _stack_batch1(S, one_token_rows, steps_batch1)
        return entry
    finally:
        S.close()
        del S
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="decode1")
    ap.add_argument("--reps", type=int, default=64, help="token batches in the rotation pool")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch8", action="store_true", help="skip the batch-8 hot/cold secondary figures")
    ap.add_argument("--primary-only", action="store_true", help="skip every secondary figure")
    ap.add_argument("--no-adaptive", action="store_true", help="skip the adaptive-residency secondary figures")
    ap.add_argument("--no-verify", action="store_true", help="skip the speculative-verify secondary figures")
    ap.add_argument("--no-gather-sweep", action="store_true", help="skip the gather-alone sweep over m")
    ap.add_argument("--no-layer-copy", action="store_true",
                    help="skip the whole-layer cold copy baseline")
    ap.add_argument("--no-direct-read", action="store_true",
                    help="skip the gather vs direct-read comparison (hot/cold decode, batch 1/8/32)")
    ap.add_argument("--no-ffn-batches", action="store_true",
                    help="skip the standalone grouped-FFN figures at batch 1/8/32")
    ap.add_argument("--no-step40", action="store_true", help="skip the 40-layer batch-32 secondary figures")
    ap.add_argument("--only", default=None,
                    help="run only this secondary figure (read_ceiling, mfma_rates, prefill8k, batch8_hotcold, direct_read, "
                         "adaptive_residency, verify, gather_sweep, layer_copy, ffn_by_batch, step40_batch32)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-layer secondary figures")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--no-mfma-rates", action="store_true", help="skip the matrix-core rate probe")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run one plain float64 copy of this many MiB (a known-size kernel for "
                         "scaling hardware byte counters)")
    a = ap.parse_args()
    keys = {"read_ceiling": "no_read_ceiling", "mfma_rates": "no_mfma_rates", "prefill8k": "no_prefill", "batch8_hotcold": "no_batch8",
            "direct_read": "no_direct_read", "adaptive_residency": "no_adaptive", "verify": "no_verify",
            "gather_sweep": "no_gather_sweep", "layer_copy": "no_layer_copy", "ffn_by_batch": "no_ffn_batches",
            "step40_batch32": "no_step40"}
    if a.only is not None:
        if a.only not in keys:
            ap.error(f"--only: unknown secondary {a.only}")
        for k, flag in keys.items():
            setattr(a, flag, k != a.only)
    if a.primary_only:
        for k in ("no_batch8", "no_adaptive", "no_verify", "no_layer_copy", "no_direct_read", "no_ffn_batches",
                  "no_step40", "no_gather_sweep", "no_prefill", "no_read_ceiling", "no_mfma_rates"):
            setattr(a, k, True)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "this layer is built and measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import moe_routed_expert_router_amd as moe  # noqa: F401  (fails loudly if libmoe.so is missing)

    if a.copy_probe_mb:
        n = a.copy_probe_mb * (1 << 20) // 8
        src = torch.ones(n, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {a.copy_probe_mb} MiB read + {a.copy_probe_mb} MiB written")
        del src, dst
    if a.workload == "step40":
        # the 40-layer step alone (for traces of that workload); the default
        # decode1 run reports it as a secondary figure
        e = measure_stack("step40", a.steps, a.warmup, not a.no_graph)
        if "skipped" in e:
            print(json.dumps({"metric": METRIC, "value": None, "skipped": e["skipped"]}), flush=True)
            return
        print(json.dumps({"metric": METRIC, "value": e["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "steps": a.steps, "warmup": a.warmup, "ms_per_step": e["ms_per_step"],
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": "step40", "layers": e["layers"],
                                                          "tokens_per_step": e["tokens_per_layer"]},
                          "step40_batch32": e}), flush=True)
        return
    log(f"[bench] workload {a.workload}: setup")
    prim = layer_figures(a.workload, a.steps, a.warmup, a.reps, not a.no_graph)
    wl = prim.pop("_wl")
    torch.cuda.empty_cache()

    extra = {}

    def secondary(key, title, fn):
        """One secondary figure; a host-side failure (say, no more pinned
        memory on this host) is recorded in its place and the run goes on."""
        log(f"[bench] secondary: {title}")
        try:
            extra[key] = fn()
        except Exception as e:   # noqa: BLE001 - reported in the JSON line
            log(f"[bench] secondary {key} failed: {type(e).__name__}: {e}")
            extra[key] = {"error": f"{type(e).__name__}: {e}"}
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    def batch8():
        f = layer_figures("hotcold8", 128, 8, 16, not a.no_graph)
        f.pop("_wl")
        return f

    def prefill():
        f = layer_figures("prefill8k", 20, 2, 2, not a.no_graph)
        f.pop("_wl")
        return f

    if a.workload == "decode1":
        if not a.no_read_ceiling:
            secondary("read_ceiling", "single-launch streaming-read ceiling (6.3 / 26.9 / 53.5 / 80.4 MB)",
                      measure_read_ceiling)
        if not a.no_mfma_rates:
            secondary("mfma_rates", "matrix-core rates: bf16 and scaled f8f6f4 forms, GPU full", measure_mfma_rates)
        if not a.no_prefill:
            secondary("prefill8k", "prefill layer (8192 tokens, all resident, grouped GEMM)", prefill)
        if not a.primary_only and a.only is None:
            secondary("host_call", "host time of one eager moe_layer_forward (decode1)", measure_host_call)
        if not a.no_batch8:
            secondary("batch8_hotcold", "hotcold8 (batch 8, 255 hot / 129 cold)", batch8)
        if not a.no_direct_read:
            secondary("direct_read", "gather-then-compute vs direct read of cold experts (batch 1/8/32)",
                      measure_direct_read)
        if not a.no_adaptive:
            secondary("adaptive_residency", "adaptive residency on drifting traffic",
                      lambda: {"drifted_once": measure_adaptive(), "drifting": measure_adaptive(drift_every=250)})
        if not a.no_verify:
            secondary("verify", "speculative-verify steps (streams x (1 + draft), correlated windows)",
                      measure_verify)
        if not a.no_gather_sweep:
            secondary("gather_sweep", "cold gather alone, m = 1..129 picked cold experts, beside DMA copies",
                      measure_gather_sweep)
        if not a.no_layer_copy:
            secondary("layer_copy", "layer-granular copy baseline (all 384 experts of a layer from the host)",
                      measure_layer_copy)
        if not a.no_ffn_batches:
            secondary("ffn_by_batch", "grouped FFN alone at batch 1/8/32 (all experts resident)",
                      measure_ffn_batches)
        if not a.no_step40:
            secondary("step40_batch32", "step40 (40 layers, batch 32, 255 hot / 129 cold, shared scratch)",
                      lambda: measure_stack("step40", 10, 2, not a.no_graph, one_token_rows=16))
            lc, st = extra.get("layer_copy"), extra["step40_batch32"]
            if lc and "tokens_per_s" in lc and "tokens_per_s" in st:
                lc["picked_only_over_layer_copy"] = round(st["tokens_per_s"] / lc["tokens_per_s"], 1)

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(a.workload, a.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": prim["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": a.workload, "hidden": wl.hidden, "inter": wl.inter, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "tokens_per_step": wl.tokens, "layers": 1,
                   "resident": "all experts in HBM" if wl.n_hot is None else f"{wl.n_hot} hot / {wl.n_cold} cold",
                   "weights": "MXFP4 (e2m1 + e8m0/32)", "accumulate": "fp32", "graph": prim["graph"],
                   "token_batches_rotated": min(a.reps, a.steps)},
        "repeats": prim["repeats"],
        "roofline": prim["roofline"],
        "ffn": prim["ffn"],
        "kernels": prim["kernels"],
        "cpu_baseline": cpu,
    }
    for k in ("down_kernel", "down_TFLOP_per_s", "layer_useful_TFLOP_per_s"):
        if k in prim:
            out[k] = prim[k]
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
