"""Test-side helpers written independently of the oracle and the GPU library."""
from fractions import Fraction
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16_bits_to_f64(a):
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v):
    """Round float64 to bf16 (nearest, ties to even) without passing through float32."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat, of = v.ravel(), out.ravel()
    m, e = np.frexp(flat)
    qexp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, qexp)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(flat / q) * q
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, flat), r)
        r = np.where(np.isnan(flat), np.nan, r)
        r = np.where(flat == 0, flat, r)
    of[:] = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    of[np.isnan(flat)] = 0x7FC0
    return out


def fraction_to_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest float32 (ties to even), integers only."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    qe = max(e - 23, -149)
    scaled = q / (Fraction(2) ** qe)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** qe
    if val >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(val)


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    s = -1 if bits >> 15 else 1
    be = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if be == 0:
        return s * Fraction(f) * Fraction(2) ** -133
    return s * Fraction(128 + f) * Fraction(2) ** (be - 134)


def e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)], dtype=np.float64)


def np_dequant(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Dequantise with numpy from the golden table: low nibble first, 32-blocks along a row."""
    lut = e2m1_table()
    c = codes.reshape(rows, cols // 2)
    nib = np.empty((rows, cols), dtype=np.int64)
    nib[:, 0::2] = c & 15
    nib[:, 1::2] = c >> 4
    s = scales.reshape(rows, cols // 32).astype(np.int64)
    sc = np.repeat(s, 32, axis=1)
    with np.errstate(over="ignore"):
        w = np.ldexp(lut[nib], sc - 127).astype(np.float32)
    w[sc == 255] = np.nan
    return w


def split_record(record: np.ndarray, L: int, F: int):
    """Slices (codes, scales) of gate [F,L], up [F,L], down [L,F] inside one expert record."""
    nc, ns = F * L // 2, F * L // 32
    mat = nc + ns
    out = []
    for m in range(3):
        base = m * mat
        out.append((record[base:base + nc], record[base + nc:base + mat]))
    return out


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def cosine(a, b) -> float:
    """Cosine similarity of two vectors, in fp64."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b)))
