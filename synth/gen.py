"""Seeded synthetic inputs: workloads, token and router arrays, MXFP4 expert
bytes, the Zipf logit prior and residency tables.

Sources of the recipe (what the web pages on the method fix, and what this
module takes for them):

* 384 routed experts per layer and top-6 routing: the GB300 "inference
  engineering" write-up (first paragraph on the mixture-of-experts design).
* Routed experts stored as MXFP4 ("expert nibbles"): the two-workstation
  V4.1-Flash report, Abstract and section 1.
* 255 hot / 129 cold experts per layer, one scratch slot per cold expert,
  40 layers sharing it: the "gracetier" write-up, section 1 ("The idea").
* 98.7% of picks landing on 73% of experts: the GB300 write-up, the
  paragraph on hot/cold doors closed by the hardware.
* Speculative verify windows: 1 + 5 tokens per stream at 1-4 streams, 1 + 1
  at 5-16 (the GB300 write-up, its launch-flag table, the speculative-config
  row); a 1 + 5 window touching 3.7x the distinct experts of one token (the
  same write-up, the table of what was tried, the speculative-fetching row).
  Tokens of one window share a common component (correlation rho, fitted to
  that multiplier with the oracle's router and kept in verify_calibration.json).

Expert weight bytes come from a counter-based 32-bit hash so that the same
bytes can be produced on the CPU (numpy, for the oracle) and directly in GPU
memory (torch integer ops, for 5-200 GB of resident experts) and agree bit
for bit.  Token activations and router weights are small and come from
numpy's Philox generator on the CPU; callers copy them to the device.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "expert_bytes", "section_sizes",
    "stream_keys", "hash_words_np", "expert_sections", "expert_blob",
    "fill_expert_blobs_device", "tokens_bf16", "router_weight", "zipf_prior",
    "load_calibration", "hot_set", "residency_slots", "bf16_round_bits",
    "CALIBRATION_PATH", "verify_window", "verify_tokens_bf16", "load_verify_calibration",
    "VERIFY_CALIBRATION_PATH", "drifted_zipf_prior",
]

M32 = 0xFFFFFFFF

# Section tags of the per-expert byte streams and of the Philox streams.
TAG_W13_NIB, TAG_W13_SCALE, TAG_W2_NIB, TAG_W2_SCALE = 1, 2, 3, 4
TAG_TOKENS, TAG_ROUTER, TAG_ZIPF_RANK = 5, 6, 7
TAG_VERIFY_SHARED, TAG_VERIFY_OWN = 8, 9
TAG_DRIFT = 10

SCALE_LO, SCALE_N = 123, 5          # e8m0 bytes uniform over 123..127 (2^-4..2^0)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  All sizes are the pages' model shapes."""
    name: str
    hidden: int          # H
    inter: int           # I (per-expert FFN width)
    n_experts: int       # E
    top_k: int           # k
    tokens: int          # T per layer
    layers: int = 1
    n_hot: int | None = None   # None: every expert resident in HBM
    zipf: bool = False         # Zipf(s=1.1) logit prior on the router
    seed: int = 0

    @property
    def n_cold(self) -> int:
        return 0 if self.n_hot is None else self.n_experts - self.n_hot

    @property
    def hot_count(self) -> int:
        return self.n_experts if self.n_hot is None else self.n_hot


WORKLOADS = {
    # tiny correctness case: 8 experts, top-2, H=256, I=128, 4 tokens
    "tiny": Workload("tiny", 256, 128, 8, 2, 4),
    # one decode token through one layer, 384 experts resident
    "decode1": Workload("decode1", 4096, 2048, 384, 6, 1),
    # 8 decode tokens, 255 hot / 129 cold, Zipf-biased routing
    "hotcold8": Workload("hotcold8", 4096, 2048, 384, 6, 8, 1, 255, True),
    # 40 sequential layers, 32 tokens, 255/129 per layer, one shared scratch
    "step40": Workload("step40", 4096, 2048, 384, 6, 32, 40, 255, True),
    # prefill: 8192 tokens, all resident, uniform prior
    "prefill8k": Workload("prefill8k", 4096, 2048, 384, 6, 8192),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# Expert blob sections (a stated convention; the oracle and the HIP library
# each read the bytes with their own code).  One contiguous blob per expert,
# four sections in this order, each filled as one keyed byte stream:
#   w13 codes   2I*H/2 bytes   e2m1, two per byte (gate rows, then up rows)
#   w13 scales  2I*H/32 bytes  e8m0, one per 32 elements along H
#   w2  codes   H*I/2 bytes    down projection, contraction along I
#   w2  scales  H*I/32 bytes
# Where a given (row, column) sits inside a section is the readers' layout
# (tiles of 16 rows x 128 columns); the generator only fills bytes.
# --------------------------------------------------------------------------
def section_sizes(H: int, I: int) -> tuple[int, int, int, int]:
    return (2 * I * H // 2, 2 * I * H // 32, H * I // 2, H * I // 32)


def expert_bytes(H: int, I: int) -> int:
    return sum(section_sizes(H, I))


# --------------------------------------------------------------------------
# Counter-based hash.  mix32 is the "lowbias32" integer finaliser published
# in C. Wellons' hash-prospector; word i of a stream keyed (k1, k2) is
# mix32(mix32(i + k1) ^ k2).  Both implementations below are exact integer
# arithmetic modulo 2^32.
# --------------------------------------------------------------------------
_C1, _C2 = 0x7FEB352D, 0x846CA68B


def _mix32_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * _C1) & M32
    x ^= x >> 15
    x = (x * _C2) & M32
    x ^= x >> 16
    return x


def stream_keys(seed: int, tag: int, layer: int, expert: int) -> tuple[int, int]:
    h = _mix32_int(seed ^ 0x243F6A88)
    h = _mix32_int(h ^ ((tag * 0x9E3779B9) & M32))
    h = _mix32_int(h ^ (((layer + 1) * 0x85EBCA6B) & M32))
    h = _mix32_int(h ^ (((expert + 1) * 0xC2B2AE35) & M32))
    return h, _mix32_int(h ^ 0x5BD1E995)


def _mix32_np(x: np.ndarray) -> np.ndarray:
    # x: uint32 array, modified in place (uint32 multiply wraps modulo 2^32)
    x ^= x >> np.uint32(16)
    x *= np.uint32(_C1)
    x ^= x >> np.uint32(15)
    x *= np.uint32(_C2)
    x ^= x >> np.uint32(16)
    return x


def hash_words_np(k1: int, k2: int, n: int, start: int = 0) -> np.ndarray:
    """Words start..start+n-1 of stream (k1, k2) as uint32."""
    i = np.arange(start, start + n, dtype=np.uint64)
    x = ((i + np.uint64(k1)) & np.uint64(M32)).astype(np.uint32)
    _mix32_np(x)
    x ^= np.uint32(k2)
    return _mix32_np(x)


def _scale_bytes_from_words(w: np.ndarray) -> np.ndarray:
    return (SCALE_LO + ((w.astype(np.uint64) * np.uint64(SCALE_N)) >> np.uint64(32))).astype(np.uint8)


def expert_sections(seed: int, layer: int, expert: int, H: int, I: int):
    """The four section byte streams (w13 codes, w13 scales, w2 codes, w2
    scales) of one expert, as flat uint8 arrays in blob order."""
    out = []
    for tag, nbytes in zip((TAG_W13_NIB, TAG_W13_SCALE, TAG_W2_NIB, TAG_W2_SCALE), section_sizes(H, I)):
        k1, k2 = stream_keys(seed, tag, layer, expert)
        if tag in (TAG_W13_NIB, TAG_W2_NIB):
            w = hash_words_np(k1, k2, nbytes // 4)
            b = w.astype("<u4").view(np.uint8)
        else:
            b = _scale_bytes_from_words(hash_words_np(k1, k2, nbytes))
        out.append(b)
    return tuple(out)


def expert_blob(seed: int, layer: int, expert: int, H: int, I: int) -> np.ndarray:
    return np.concatenate(expert_sections(seed, layer, expert, H, I))


# ---------------------------- GPU-side generation ---------------------------
def _mul32_t(x, c: int):
    # (x * c) mod 2^32 for 0 <= x < 2^32 held in int64, without overflow
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32


def _mix32_t(x):
    x = x ^ (x >> 16)
    x = _mul32_t(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32_t(x, _C2)
    return x ^ (x >> 16)


def _hash_words_t(k1, k2, n: int, start: int, device):
    """k1, k2: int64 tensors [m, 1]; returns int64 [m, n] of words in [0, 2^32)."""
    import torch
    i = torch.arange(start, start + n, dtype=torch.int64, device=device).unsqueeze(0)
    x = (i + k1) & M32
    x = _mix32_t(x)
    x = x ^ k2
    return _mix32_t(x)


def fill_expert_blobs_device(out, seed: int, layer: int, experts: Sequence[int], H: int, I: int,
                             chunk_words: int = 1 << 24) -> None:
    """Write the blobs of `experts` into rows of `out` (torch uint8 [len(experts)][B],
    any device) bit-identically to expert_blob()."""
    import torch
    dev = out.device
    B = expert_bytes(H, I)
    assert out.dtype == torch.uint8 and out.dim() == 2 and out.shape[1] == B
    assert out.shape[0] == len(experts)
    sizes = section_sizes(H, I)
    offs = np.cumsum((0,) + sizes)
    tags = (TAG_W13_NIB, TAG_W13_SCALE, TAG_W2_NIB, TAG_W2_SCALE)
    experts = list(experts)
    for si, tag in enumerate(tags):
        nib = tag in (TAG_W13_NIB, TAG_W2_NIB)
        nwords = sizes[si] // 4 if nib else sizes[si]
        per = max(1, min(len(experts), chunk_words // max(1, nwords)))
        for e0 in range(0, len(experts), per):
            grp = experts[e0:e0 + per]
            keys = [stream_keys(seed, tag, layer, e) for e in grp]
            k1 = torch.tensor([k[0] for k in keys], dtype=torch.int64, device=dev).unsqueeze(1)
            k2 = torch.tensor([k[1] for k in keys], dtype=torch.int64, device=dev).unsqueeze(1)
            step = max(1, chunk_words // len(grp))
            for w0 in range(0, nwords, step):
                n = min(step, nwords - w0)
                w = _hash_words_t(k1, k2, n, w0, dev)
                dst = out[e0:e0 + len(grp), offs[si]:offs[si + 1]]
                if nib:
                    w32 = torch.where(w >= (1 << 31), w - (1 << 32), w).to(torch.int32)
                    dst[:, 4 * w0:4 * (w0 + n)] = w32.view(torch.uint8).view(len(grp), 4 * n)
                else:
                    dst[:, w0:w0 + n] = (SCALE_LO + ((w * SCALE_N) >> 32)).to(torch.uint8)
                del w


# ------------------------------ small arrays --------------------------------
def _philox(seed: int, tag: int, layer: int) -> np.random.Generator:
    k1, k2 = stream_keys(seed, tag, layer, 0)
    return np.random.Generator(np.random.Philox(key=(k1 << 32) | k2))


def bf16_round_bits(f: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def tokens_bf16(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    """Activations x ~ N(0,1) rounded to bf16; returned as uint16 bits [T][H]."""
    g = _philox(seed, TAG_TOKENS, layer)
    return bf16_round_bits(g.standard_normal((T, H), dtype=np.float32))


def router_weight(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    """Router matrix Wr ~ N(0, 0.02^2), fp32 [E][H]."""
    g = _philox(seed, TAG_ROUTER, layer)
    return (g.standard_normal((E, H), dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def zipf_prior(seed: int, layer: int, E: int, alpha: float, s: float = 1.1) -> np.ndarray:
    """Logit prior b_e = -alpha * s * ln(rank_e), ranks a seeded permutation of 1..E."""
    g = _philox(seed, TAG_ZIPF_RANK, layer)
    rank = g.permutation(E).astype(np.float64) + 1.0
    return (-alpha * s * np.log(rank)).astype(np.float32)


def verify_window(streams: int) -> int:
    """Tokens per stream in one verify step: the drafter proposes 5 tokens
    at 1-4 concurrent streams and 1 at 5-16, and the step checks them with
    the stream's current token (1 + draft length)."""
    if not 1 <= streams <= 16:
        raise ValueError("the draft schedule covers 1..16 streams")
    return 6 if streams <= 4 else 2


def verify_tokens_bf16(seed: int, layer: int, streams: int, window: int, H: int, rho: float) -> np.ndarray:
    """Verify-step activations, uint16 bf16 bits [streams*window][H], rows
    stream-major.  Row (s, j) = sqrt(rho) * a_s + sqrt(1 - rho) * n_sj with
    a_s, n_sj ~ N(0, I) drawn independently: unit variance per element,
    correlation rho between two tokens of one window, none across windows."""
    a = _philox(seed, TAG_VERIFY_SHARED, layer).standard_normal((streams, H), dtype=np.float32)
    n = _philox(seed, TAG_VERIFY_OWN, layer).standard_normal((streams, window, H), dtype=np.float32)
    x = np.float32(math.sqrt(rho)) * a[:, None, :] + np.float32(math.sqrt(1.0 - rho)) * n
    return bf16_round_bits(x.reshape(streams * window, H))


def drifted_zipf_prior(seed: int, layer: int, E: int, alpha: float, frac: float, rounds: int,
                       s: float = 1.1) -> np.ndarray:
    """zipf_prior after `rounds` rounds of drift: each round takes round(frac*E)
    random positions of the rank permutation and shuffles their ranks among
    themselves (traffic whose favourite experts differ from the calibration's;
    rounds = 0 is zipf_prior itself)."""
    g = _philox(seed, TAG_ZIPF_RANK, layer)
    rank = g.permutation(E).astype(np.float64) + 1.0
    m = int(round(frac * E))
    for r in range(rounds):
        k1, k2 = stream_keys(seed, TAG_DRIFT, layer, r)
        d = np.random.Generator(np.random.Philox(key=(k1 << 32) | k2))
        pos = d.choice(E, m, replace=False)
        rank[pos] = rank[d.permutation(pos)]
    return (-alpha * s * np.log(rank)).astype(np.float32)


# ----------------------------- calibration data -----------------------------
CALIBRATION_PATH = os.path.join(os.path.dirname(__file__), "zipf_calibration.json")


def load_calibration(path: str = CALIBRATION_PATH) -> dict:
    with open(path) as f:
        return json.load(f)


VERIFY_CALIBRATION_PATH = os.path.join(os.path.dirname(__file__), "verify_calibration.json")


def load_verify_calibration(path: str = VERIFY_CALIBRATION_PATH) -> dict:
    with open(path) as f:
        return json.load(f)


def hot_set(seed: int, layer: int, cal: dict | None = None) -> list[int]:
    """The 255 most-picked experts of (seed, layer) in the calibration sample."""
    cal = cal or load_calibration()
    return list(cal["hot"][f"{seed}:{layer}"])


def residency_slots(hot: Iterable[int], E: int) -> np.ndarray:
    """Residency table slot[E] (int32): hot experts, in ascending expert order,
    get HBM indices 0..n_hot-1 (slot >= 0); cold experts, in ascending order,
    get scratch / host slots c = 0..n_cold-1 stored as slot = -c-1."""
    hot = set(int(e) for e in hot)
    slot = np.empty(E, dtype=np.int32)
    h = c = 0
    for e in range(E):
        if e in hot:
            slot[e] = h
            h += 1
        else:
            slot[e] = -c - 1
            c += 1
    return slot
