"""Device-side setup of a synthetic layer for the GPU tests and the bench.

Allocates (torch) and fills one layer's inputs: tokens, router, Zipf prior,
hot experts in HBM, cold experts in pinned host memory mapped for the GPU
(moe_host_alloc), a cold scratch, the residency table and a workspace.  Expert
bytes are generated directly in device memory with synth's GPU generator,
which reproduces synth.expert_blob (the oracle's source) bit for bit.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import moe_routed_expert_router_amd as moe
from synth import gen


class HostBuffer:
    """Pinned, device-mapped host memory from the library; freed on close()."""

    def __init__(self, nbytes: int, coherent: bool = False):
        self.nbytes = nbytes
        self.host, self.dev = moe.moe_host_alloc(nbytes, coherent)
        arr_t = ctypes.c_uint8 * nbytes
        self.np = np.frombuffer(arr_t.from_address(self.host), dtype=np.uint8)

    def close(self):
        if self.host:
            self.np = None
            moe.moe_host_free(self.host)
            self.host = self.dev = 0


def fill_host_experts(buf: HostBuffer, seed: int, layer: int, experts, H: int, I: int, chunk: int = 16):
    """Write the blobs of `experts` (in order) into consecutive slots of buf."""
    B = gen.expert_bytes(H, I)
    experts = list(experts)
    view = buf.np[: len(experts) * B].reshape(len(experts), B)
    for i in range(0, len(experts), chunk):
        grp = experts[i:i + chunk]
        tmp = torch.empty((len(grp), B), dtype=torch.uint8, device="cuda")
        gen.fill_expert_blobs_device(tmp, seed, layer, grp, H, I)
        view[i:i + len(grp)] = tmp.cpu().numpy()
        del tmp


class Layer:
    """One layer of a workload, resident as the workload says."""

    def __init__(self, wl: gen.Workload, layer: int = 0, T: int | None = None, scratch=None,
                 all_hot: bool = False, cal: dict | None = None, coherent: bool = False,
                 hot: list | None = None, host: HostBuffer | None = None, direct: bool = False,
                 x_np: np.ndarray | None = None):
        """direct: cold experts are read in place from the pinned host pool
        (the residency's scratch is the host pool; nothing is gathered).
        x_np: the tokens (uint16 bf16 bits [T][H]) instead of the seeded N(0,1) ones."""
        self.wl, self.layer = wl, layer
        H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
        self.H, self.I, self.E, self.k = H, I, E, k
        self.T = (wl.tokens if T is None else T) if x_np is None else x_np.shape[0]
        self.B = gen.expert_bytes(H, I)
        self.shape = moe.shape(H, I, E, k)
        seed = wl.seed
        self.x_np = gen.tokens_bf16(seed, layer, self.T, H) if x_np is None else np.ascontiguousarray(x_np)
        self.wr_np = gen.router_weight(seed, layer, E, H)
        self.bias_np = None
        if wl.zipf:
            cal = cal or gen.load_calibration()
            self.bias_np = gen.zipf_prior(seed, layer, E, cal["alpha"])
        if hot is not None:
            hot = list(hot)
        elif wl.n_hot is None or all_hot:
            hot = list(range(E))
        else:
            hot = gen.hot_set(seed, layer, cal)
        self.slot_np = gen.residency_slots(hot, E)
        self.hot = [e for e in range(E) if self.slot_np[e] >= 0]
        self.cold = [e for e in range(E) if self.slot_np[e] < 0]
        self.n_hot, self.n_cold = len(self.hot), len(self.cold)

        dev = "cuda"
        self.x = torch.from_numpy(self.x_np.view(np.int16)).to(dev)
        self.wr = torch.from_numpy(self.wr_np).to(dev)
        self.bias = torch.from_numpy(self.bias_np).to(dev) if self.bias_np is not None else None
        self.slot = torch.from_numpy(self.slot_np).to(dev)
        self.hot_base = torch.empty((max(self.n_hot, 1), self.B), dtype=torch.uint8, device=dev)
        if self.n_hot:
            gen.fill_expert_blobs_device(self.hot_base, seed, layer, self.hot, H, I)
        self.host = None
        self.own_host = host is None   # a borrowed pool keeps another layer's bytes
        self.scratch = None
        if self.n_cold:
            if host is None:
                self.host = HostBuffer(self.n_cold * self.B, coherent)
                fill_host_experts(self.host, seed, layer, self.cold, H, I)
            else:
                assert host.nbytes == self.n_cold * self.B
                self.host = host
            if not direct:
                self.scratch = scratch if scratch is not None else torch.empty(
                    (self.n_cold, self.B), dtype=torch.uint8, device=dev)
        self.direct = direct and self.n_cold > 0
        self.residency = moe.residency(self.slot, self.hot_base if self.n_hot else None,
                                       self.host.dev if self.host else None,
                                       self.host.dev if self.direct else self.scratch,
                                       self.n_hot, self.n_cold)
        self.ws = torch.empty(moe.moe_workspace_bytes(self.shape, self.T), dtype=torch.uint8, device=dev)
        self.ids = torch.empty((self.T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((self.T, k), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.T, H), dtype=torch.float32, device=dev)

    def blob(self, e: int) -> np.ndarray:
        """The oracle's copy of expert e (regenerated on the CPU by synth)."""
        return gen.expert_blob(self.wl.seed, self.layer, e, self.H, self.I)

    def forward(self, out_bf16: bool = False, stream=None):
        out = self.out if not out_bf16 else torch.empty((self.T, self.H), dtype=torch.bfloat16, device="cuda")
        moe.moe_layer_forward(self.shape, self.x, self.wr, self.bias, True, self.residency, self.ids, self.w,
                              out, self.ws, stream)
        return out

    def close(self):
        if self.host and self.own_host:
            self.host.close()
        self.host = None


class Stack:
    """`layers` sequential layers of a workload (each with its own seeded
    tokens, router, Zipf prior, hot pool and pinned cold pool) sharing one
    cold scratch, run in order on one stream.  Tokens are independent per
    layer (an unnormalised synthetic layer's output is not a usable input)."""

    def __init__(self, wl: gen.Workload, layers: int | None = None, T: int | None = None, log=None,
                 share_host_on_oom: bool = False, max_host_pools: int | None = None):
        cal = gen.load_calibration() if wl.zipf else None
        n = wl.layers if layers is None else layers
        B = gen.expert_bytes(wl.hidden, wl.inter)
        self.scratch = torch.empty((max(wl.n_cold, 1), B), dtype=torch.uint8, device="cuda")
        self.layers = []
        self.distinct_host_pools = 0
        try:
            for l in range(n):
                L = None
                if max_host_pools is None or self.distinct_host_pools < max_host_pools:
                    try:
                        L = Layer(wl, layer=l, T=T, scratch=self.scratch, cal=cal)
                    except moe.MoeError:
                        if not share_host_on_oom or not self.distinct_host_pools:
                            raise
                if L is None:
                    # no (more) pinned host memory: reuse an earlier layer's cold pool
                    # (same host-link traffic; that layer's bytes, not this one's)
                    donor = self.layers[l % self.distinct_host_pools]
                    L = Layer(wl, layer=l, T=T, scratch=self.scratch, cal=cal, host=donor.host)
                self.distinct_host_pools += int(L.own_host)
                self.layers.append(L)
                if log and (l % 10 == 9 or l == n - 1):
                    log(f"[setup] {l + 1}/{n} layers resident, {self.distinct_host_pools} distinct cold pools")
        except Exception:
            self.close()
            raise
        self.wl = wl

    def forward(self, stream=None):
        for L in self.layers:
            L.forward(stream=stream)

    def close(self):
        for L in self.layers:
            L.close()
        self.layers = []
