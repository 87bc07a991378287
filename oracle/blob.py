"""Per-expert byte layout.

Test infrastructure: only tests/, the bench's CPU baseline and the smoke
check use this package.

The "gracetier" write-up (section 1) copies whole cold experts into their
scratch slots, so each expert is one contiguous blob.  The offloaded planes
are named w13 (gate and up fused) and w2 (down) in the GB300 write-up's flag
table (the --cpu-offload-params row).  The pages fix the number format
(MXFP4: e2m1 codes, an e8m0 scale per 32 elements; two-workstation report,
Abstract and section 1) but not where the bytes sit; the layout taken here:

  w13 codes   (2I x H)   rows 0..I-1 are the gate projection, I..2I-1 up
  w13 scales
  w2  codes   (H x I)    down projection, contraction along I
  w2  scales

in that order, each plane of R rows and K columns (MX blocks of 32 along K)
stored in tiles of 16 rows x 128 columns: with nst = K / 128, the codes of
row r, column c (two per byte, c even in the low nibble) are byte

  ((r // 16) * nst + c // 128) * 1024 + (r % 16) * 64 + (c % 128) // 2

of the codes section, and the scale of row r, block b = c // 32 is byte

  ((r // 16) * nst + b // 4) * 64 + (r % 16) * 4 + b % 4

of the scales section.  Total 3*H*I*17/32 bytes (13,369,344 at H=4096,
I=2048).  split() returns the planes as row-major matrices (copies); join()
is its inverse.
"""
import numpy as np

from .mx import dequant


def sizes(H, I):
    """Byte sizes of the four sections, in blob order."""
    return (2 * I * (H // 2), 2 * I * (H // 32), H * (I // 2), H * (I // 32))


def blob_bytes(H, I):
    return sum(sizes(H, I))


def _untile(sec, R, per_row, per_tile):
    """Tiled section -> row-major [R][per_row]: 16-row groups, tiles of
    per_tile bytes per row, groups stored tile after tile."""
    nst = per_row // per_tile
    return sec.reshape(R // 16, nst, 16, per_tile).transpose(0, 2, 1, 3).reshape(R, per_row)


def _tile(mat, per_tile):
    """Row-major [R][per_row] -> tiled section bytes (inverse of _untile)."""
    R, per_row = mat.shape
    nst = per_row // per_tile
    return np.ascontiguousarray(mat.reshape(R // 16, 16, nst, per_tile).transpose(0, 2, 1, 3)).reshape(-1)


def split(blob, H, I):
    """blob uint8 [B] -> row-major copies (w13 codes [2I][H/2], w13 scales
    [2I][H/32], w2 codes [H][I/2], w2 scales [H][I/32])."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    assert blob.size == blob_bytes(H, I), (blob.size, blob_bytes(H, I))
    assert H % 128 == 0 and I % 128 == 0, (H, I)
    o = np.cumsum((0,) + sizes(H, I))
    w13q = _untile(blob[o[0]:o[1]], 2 * I, H // 2, 64)
    w13s = _untile(blob[o[1]:o[2]], 2 * I, H // 32, 4)
    w2q = _untile(blob[o[2]:o[3]], H, I // 2, 64)
    w2s = _untile(blob[o[3]:o[4]], H, I // 32, 4)
    return w13q, w13s, w2q, w2s


def join(w13q, w13s, w2q, w2s):
    """Row-major planes (as split returns them) -> blob uint8 [B]."""
    parts = [np.asarray(a, dtype=np.uint8) for a in (w13q, w13s, w2q, w2s)]
    return np.concatenate([_tile(parts[0], 64), _tile(parts[1], 4), _tile(parts[2], 64), _tile(parts[3], 4)])


def weights(blob, H, I):
    """(W13 [2I][H], W2 [H][I]) dequantised in float64 (exact)."""
    w13q, w13s, w2q, w2s = split(blob, H, I)
    return dequant(w13q, w13s), dequant(w2q, w2s)
