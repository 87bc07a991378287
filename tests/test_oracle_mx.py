"""Pins for oracle.mx and oracle.blob: MXFP4 decoding and the expert layout.

Against: the OCP MX v1.0 FP4/E8M0 tables (tests/golden), IEEE-754 bit fields,
hand-packed bytes, and the generator's independent section writer."""
import math
import os
import struct

import numpy as np
import pytest

from oracle import blob, mx
from synth import gen
from tests.brute import E2M1, GOLDEN

def test_e2m1_matches_ocp_table():
    got = mx.e2m1_value(np.arange(16))
    for code in range(16):
        assert got[code] == E2M1[code], code
        # the sign of zero is part of the table (1000 is -0.0)
        assert math.copysign(1.0, got[code]) == math.copysign(1.0, E2M1[code])


def _golden_e8m0():
    rows = []
    with open(os.path.join(GOLDEN, "ocp_mx_e8m0.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                b, v = line.split()
                rows.append((int(b), v))
    return rows


def test_e8m0_named_values():
    for b, v in _golden_e8m0():
        got = float(mx.e8m0_value(b))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, int(v[2:])), (b, v)


def test_e8m0_float64_bit_fields():
    # every non-NaN scale is a power of two: float64 exponent field = b-127+1023,
    # mantissa field 0 (checked on the raw bits, not by recomputing 2**n)
    vals = mx.e8m0_value(np.arange(255))
    for b in range(255):
        bits = struct.unpack("<Q", struct.pack("<d", float(vals[b])))[0]
        assert bits & ((1 << 52) - 1) == 0, b
        assert (bits >> 52) & 0x7FF == b - 127 + 1023, b
        assert bits >> 63 == 0
    assert np.all(vals[1:] == 2 * vals[:-1])


def test_nibble_order_hand_packed():
    # 0x21: low nibble 1 (element 0 = 0.5), high nibble 2 (element 1 = 1.0)
    # 0xF0: low nibble 0 (element 2 = 0.0), high nibble 15 (element 3 = -6.0)
    codes = mx.unpack_codes(np.array([[0x21, 0xF0]], dtype=np.uint8))
    assert codes.tolist() == [[1, 2, 0, 15]]


def test_dequant_exhaustive_codes_and_scales():
    # every (code, scale byte) pair: element = table[code] * 2^(s-127)
    codes = np.arange(16)
    packed_row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)    # 8 bytes
    packed = np.zeros((256, 16), dtype=np.uint8)
    packed[:, :8] = packed_row
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w = mx.dequant(packed, scales)
    for s in range(256):
        for c in range(16):
            v = w[s, c]
            if s == 255:
                assert math.isnan(v)
            else:
                assert v == math.ldexp(E2M1[c], s - 127), (s, c)


def test_dequant_block_boundary():
    # K = 64: columns 0..31 use scale 0, 32..63 use scale 1
    packed = np.full((1, 32), 0x22, dtype=np.uint8)        # every element code 2 = 1.0
    scales = np.array([[127, 130]], dtype=np.uint8)        # 1.0 and 8.0
    w = mx.dequant(packed, scales)
    assert np.all(w[0, :32] == 1.0) and np.all(w[0, 32:] == 8.0)


@pytest.mark.parametrize("H,I,expect", [
    (256, 128, (32768, 2048, 16384, 1024, 52224)),
    (4096, 2048, (8388608, 524288, 4194304, 262144, 13369344)),
])
def test_blob_sizes(H, I, expect):
    s = blob.sizes(H, I)
    assert s == expect[:4]
    assert blob.blob_bytes(H, I) == expect[4] == 3 * H * I * 17 // 32


def test_blob_split_reads_the_tiled_layout_by_brute_force():
    """Every code and scale of split() against the tile formula evaluated
    element by element on the generator's section streams (16-row x
    128-column tiles; 1 KB of codes and 64 B of scales per tile)."""
    H, I = 256, 128
    secs = gen.expert_sections(7, 2, 5, H, I)
    b = gen.expert_blob(7, 2, 5, H, I)
    got = blob.split(b, H, I)
    for plane, (R, K) in ((0, (2 * I, H)), (1, (H, I))):
        codes, scales = got[2 * plane], got[2 * plane + 1]
        csec, ssec = secs[2 * plane], secs[2 * plane + 1]
        assert codes.shape == (R, K // 2) and scales.shape == (R, K // 32)
        nst = K // 128
        for r in range(R):
            for cb in range(K // 2):          # code byte cb holds columns 2cb, 2cb+1
                tile = (r // 16) * nst + (2 * cb) // 128
                assert codes[r, cb] == csec[tile * 1024 + (r % 16) * 64 + cb % 64]
            for sb in range(K // 32):
                tile = (r // 16) * nst + sb // 4
                assert scales[r, sb] == ssec[tile * 64 + (r % 16) * 4 + sb % 4]


def test_blob_join_inverts_split():
    H, I = 384, 256
    b = gen.expert_blob(3, 1, 2, H, I)
    assert np.array_equal(blob.join(*blob.split(b, H, I)), b)
    # and a planted byte lands where the layout says: row 21, code byte 70 of w2
    w13q, w13s, w2q, w2s = blob.split(b, H, I)
    w2q[21, 70] ^= 0xFF
    b2 = blob.join(w13q, w13s, w2q, w2s)
    diff = np.flatnonzero(b2 != b)
    off = sum(blob.sizes(H, I)[:2]) + ((21 // 16) * (I // 128) + 70 // 64) * 1024 + (21 % 16) * 64 + 70 % 64
    assert diff.tolist() == [off]


def test_generator_scale_bytes_in_range():
    secs = gen.expert_sections(0, 0, 0, 256, 128)
    for sc in (secs[1], secs[3]):
        assert sc.min() >= 123 and sc.max() <= 127
        assert set(np.unique(sc)) == {123, 124, 125, 126, 127}
