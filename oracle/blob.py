"""Per-expert byte layout.

The "gracetier" write-up (section 1) copies whole cold experts into their
scratch slots, so each expert is one contiguous blob.  The offloaded planes
are named w13 (gate and up fused) and w2 (down) in the GB300 write-up's flag
table (the --cpu-offload-params row).  Layout taken (row-major, contraction
axis last, MX blocks of 32 along it):

  w13 codes   [2I][H/2]   rows 0..I-1 are the gate projection, I..2I-1 up
  w13 scales  [2I][H/32]
  w2  codes   [H][I/2]    down projection, contraction along I
  w2  scales  [H][I/32]

Total 3*H*I*17/32 bytes (13,369,344 at H=4096, I=2048).
"""
import numpy as np

from .mx import dequant


def sizes(H, I):
    """Byte sizes of the four sections, in blob order."""
    return (2 * I * (H // 2), 2 * I * (H // 32), H * (I // 2), H * (I // 32))


def blob_bytes(H, I):
    return sum(sizes(H, I))


def split(blob, H, I):
    """blob uint8 [B] -> (w13 codes, w13 scales, w2 codes, w2 scales) views."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    assert blob.size == blob_bytes(H, I), (blob.size, blob_bytes(H, I))
    s = sizes(H, I)
    o = np.cumsum((0,) + s)
    w13q = blob[o[0]:o[1]].reshape(2 * I, H // 2)
    w13s = blob[o[1]:o[2]].reshape(2 * I, H // 32)
    w2q = blob[o[2]:o[3]].reshape(H, I // 2)
    w2s = blob[o[3]:o[4]].reshape(H, I // 32)
    return w13q, w13s, w2q, w2s


def weights(blob, H, I):
    """(W13 [2I][H], W2 [H][I]) dequantised in float64 (exact)."""
    w13q, w13s, w2q, w2s = split(blob, H, I)
    return dequant(w13q, w13s), dequant(w2q, w2s)
