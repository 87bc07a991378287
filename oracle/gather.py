"""Pick set and the cold-expert gather.

The gracetier write-up, section 1: the 129 cold experts of each layer sit in
pinned host memory that the GPU reads directly; the GPU keeps one scratch area
with a slot for each cold expert, shared by all 40 layers; in each layer one
small kernel looks at the router's picks and copies just the picked cold ones
into their slots, after which all 384 experts run as if resident.

Readings taken: an expert is cold when its residency entry is negative, slot
= -entry-1, and its bytes sit at host_cold[slot]; it is copied whole, once
per layer however many tokens picked it, into scratch[slot]; unpicked slots
keep whatever they held.
"""
import numpy as np


def pick_counts(ids, n_experts):
    """Number of (token, pick) pairs routed to each expert ([E] int64)."""
    return np.bincount(np.asarray(ids).reshape(-1), minlength=n_experts)


def picked(ids):
    """Distinct picked experts in increasing order."""
    return np.unique(np.asarray(ids).reshape(-1))


def picked_cold(ids, slot):
    """Distinct picked experts whose residency entry marks them cold, increasing."""
    slot = np.asarray(slot)
    return np.array([e for e in picked(ids) if slot[e] < 0], dtype=np.int64)


def gather_cold(ids, slot, host_cold, scratch):
    """Scratch contents after the gather: host_cold [n_cold][B] and scratch
    [n_cold][B] uint8; returns a new array, rows of picked cold experts copied."""
    out = np.array(scratch, dtype=np.uint8, copy=True)
    for e in picked_cold(ids, slot):
        c = -int(slot[e]) - 1
        out[c] = host_cold[c]
    return out
