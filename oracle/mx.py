"""MXFP4 decoding.

The pages only name the format: the routed experts of V4.1-Flash ship in
"MXFP4, a 4-bit block floating-point format" with the "expert nibbles" as the
native layout (two-workstation report, Abstract and section 1).  The element
and scale encodings follow the OCP Microscaling (MX) v1.0 definition: each
element is an FP4 E2M1 code (1 sign bit, 2 exponent bits with bias 1, 1
mantissa bit, no inf/NaN), and each block of 32 consecutive elements along
the contraction axis shares one E8M0 scale (an 8-bit biased exponent, bias
127, with 0xFF meaning NaN).  Reading taken for the packing: two codes per
byte, the even-indexed element in the low nibble.
"""
import numpy as np


def e2m1_value(code):
    """Value of FP4 E2M1 code(s) 0..15, decoded from the bit fields (float64)."""
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    # exponent field 0 is subnormal: 0.man * 2^(1-bias) with bias 1
    sub = man * 0.5
    normal = np.ldexp(1.0 + man * 0.5, exp - 1)
    mag = np.where(exp == 0, sub, normal)
    return np.where(sign == 1, -mag, mag)


def e8m0_value(byte):
    """Value of E8M0 scale byte(s): 2^(byte-127); byte 255 is NaN (float64)."""
    byte = np.asarray(byte, dtype=np.int64)
    val = np.ldexp(np.ones(byte.shape), byte - 127)
    return np.where(byte == 255, np.nan, val)


def unpack_codes(packed):
    """uint8 [R][K/2] -> int codes [R][K]; element 2c in the low nibble of byte c."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, half = packed.shape
    codes = np.empty((R, 2 * half), dtype=np.int64)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def dequant(packed, scales, block=32):
    """Dequantised matrix W [R][K] (float64, exact) from nibbles [R][K/2] and
    scales [R][K/32]: W[r][c] = e2m1(code[r][c]) * e8m0(scale[r][c // 32])."""
    codes = unpack_codes(packed)
    R, K = codes.shape
    scales = np.asarray(scales, dtype=np.uint8)
    assert scales.shape == (R, K // block), (scales.shape, R, K)
    elem = e2m1_value(codes)
    scale = np.repeat(e8m0_value(scales), block, axis=1)
    return elem * scale
