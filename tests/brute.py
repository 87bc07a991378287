"""Brute-force scalar references for pinning the oracle on tiny inputs.

Written independently of oracle/: element values come from the OCP MX table
fixture, byte offsets are recomputed here, logits are exact rationals, top-k
is a search over all k-subsets, and the FFN is scalar loops in float64.
Pure Python: use only on tiny shapes.
"""
import itertools
import math
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_e2m1_table():
    table = {}
    with open(os.path.join(GOLDEN, "ocp_mx_fp4_e2m1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            table[int(code, 2)] = float(val)
    assert len(table) == 16
    return table


E2M1 = load_e2m1_table()


def bf16_value(bits):
    """Exact value of a bf16 bit pattern as a Fraction (finite patterns)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        v = Fraction(m, 128) * Fraction(2) ** (-126)
    else:
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return sign * v


def weight(blob, H, I, plane, r, c):
    """Dequantised element (row r, column c) of plane 'w13' ([2I][H]) or 'w2'
    ([H][I]), read byte by byte from the expert blob (planes in tiles of 16
    rows x 128 columns: 1 KB of codes and 64 B of scales per tile)."""
    n13 = 2 * I * H // 2
    s13 = 2 * I * H // 32
    n2 = H * I // 2
    if plane == "w13":
        K, nib_off, sc_off = H, 0, n13
    else:
        K, nib_off, sc_off = I, n13 + s13, n13 + s13 + n2
    tile = (r // 16) * (K // 128) + c // 128
    byte = int(blob[nib_off + tile * 1024 + (r % 16) * 64 + (c % 128) // 2])
    code = (byte >> 4) if (c % 2) else (byte & 0xF)
    sbyte = int(blob[sc_off + tile * 64 + (r % 16) * 4 + (c % 128) // 32])
    if sbyte == 255:
        return float("nan")
    return math.ldexp(E2M1[code], sbyte - 127)


def exact_logits(x_bits_row, wr, bias=None):
    """z_e = sum_h x_h Wr[e,h] (+ b_e) as exact Fractions for one token."""
    xs = [bf16_value(int(b)) for b in x_bits_row]
    out = []
    for e in range(len(wr)):
        s = sum((xs[h] * Fraction(float(wr[e][h])) for h in range(len(xs))), Fraction(0))
        if bias is not None:
            s += Fraction(float(bias[e]))
        out.append(s)
    return out


def topk_bruteforce(z, k):
    """Among all k-subsets with the largest sum of z, the lexicographically
    smallest index set; listed by decreasing z, ties by increasing index."""
    best, best_sum = None, None
    for s in itertools.combinations(range(len(z)), k):   # lexicographic order
        tot = sum(z[i] for i in s)
        if best_sum is None or tot > best_sum:
            best, best_sum = s, tot
    return sorted(best, key=lambda i: (-z[i], i))


def softmax_weights(z, ids, renormalize=True):
    zf = [float(v) for v in z]
    m = max(zf)
    p = [math.exp(v - m) for v in zf]
    den = sum(p[i] for i in ids) if renormalize else sum(p)
    return [p[i] / den for i in ids]


def expert_ffn_scalar(x, blob, H, I):
    """y = W2 (silu(W1 x) * W3 x) for one token x (list of H floats), float64."""
    w1 = [[weight(blob, H, I, "w13", j, c) for c in range(H)] for j in range(I)]
    w3 = [[weight(blob, H, I, "w13", I + j, c) for c in range(H)] for j in range(I)]
    w2 = [[weight(blob, H, I, "w2", r, j) for j in range(I)] for r in range(H)]
    h = []
    for j in range(I):
        g = math.fsum(w1[j][c] * x[c] for c in range(H))
        u = math.fsum(w3[j][c] * x[c] for c in range(H))
        sg = g / (1.0 + math.exp(-g)) if g > -700 else 0.0
        h.append(sg * u)
    return [math.fsum(w2[r][j] * h[j] for j in range(I)) for r in range(H)]
