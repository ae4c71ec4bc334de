"""Pins of the oracle's MXFP8-activation mode (E4M3 elements, e8m0 block scale,
OCP Microscaling v1.0 convention), which the hardware deep-dive blog's QAT section
names for the activations and the pages leave otherwise unspecified."""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from _util import GOLDEN, bf16_bits_to_f64, f64_to_bf16_bits, np_dequant, split_record


def _golden_e4m3():
    out = {}
    with open(os.path.join(GOLDEN, "e4m3_values.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                out[int(c, 16)] = float(v)
    return out


def test_e4m3_values_match_format_definition():
    for code, want in _golden_e4m3().items():
        got = oracle.e4m3_value(code)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), hex(code)


def test_e4m3_codes_ordered_and_counted():
    """Codes 0x00..0x7e increase strictly (a sign-magnitude format) and are the negatives
    of 0x80..0xfe; 254 finite codes, two NaNs."""
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    for c in range(0x7F):
        assert oracle.e4m3_value(0x80 | c) == -pos[c]
    assert sum(math.isnan(oracle.e4m3_value(c)) for c in range(256)) == 2


def _brute_block(v):
    """MXFP8 of 32 values by search: the scale from the definition, then for each
    element the nearest finite E4M3 value (ties: even code), which saturates by itself."""
    v = np.asarray(v, dtype=np.float64)
    amax = float(np.max(np.abs(v)))
    if amax == 0.0:
        X = -127
    else:
        X = max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
    vals = {c: oracle.e4m3_value(c) for c in range(256) if not math.isnan(oracle.e4m3_value(c))}
    codes = []
    for x in v:
        t = math.ldexp(float(x), -X)
        neg = math.copysign(1.0, t) < 0
        cands = [c for c in vals if (c >= 0x80) == neg]
        best = min(cands, key=lambda c: (abs(t - vals[c]), c & 1))
        codes.append(best)
    return np.array(codes, dtype=np.uint8), X + 127


@pytest.mark.parametrize("seed", range(8))
def test_mxfp8_block_matches_nearest_value_search(seed):
    rng = np.random.default_rng(seed)
    scale = 10.0 ** rng.uniform(-6, 6)
    v = rng.standard_normal(32) * scale
    if seed % 2:
        v[rng.integers(32)] = 0.0
    if seed % 3 == 0:
        v = -np.abs(v)
    codes, sc = oracle.mxfp8_block(v)
    bcodes, bsc = _brute_block(v)
    assert sc == bsc and np.array_equal(codes, bcodes)


def test_mxfp8_block_special_cases():
    # all ones: X = -8, every element 1 * 2^8 = 256 = code 0x78
    c, s = oracle.mxfp8_block(np.ones(32))
    assert s == 119 and (c == 0x78).all()
    # a tie: with max 1.0 (X = -8), 136/256 scales to 136, halfway between 128 (even
    # mantissa) and 144, and rounds to 128 = code 0x70
    v = np.zeros(32)
    v[0], v[1] = 1.0, 136.0 / 256.0
    c, s = oracle.mxfp8_block(v)
    assert s == 119 and c[1] == 0x70 and oracle.e4m3_value(int(c[1])) == 128.0
    # saturation: 1.9 scales to 486.4 > 448
    v[0] = 1.9
    c, _ = oracle.mxfp8_block(v)
    assert c[0] == 0x7E
    # an E4M3 subnormal: 2^-16 with max 1.0 scales to 2^-8 = 2 * 2^-9
    v[0], v[1] = 1.0, 2.0 ** -16
    c, _ = oracle.mxfp8_block(v)
    assert c[1] == 0x02
    # zeros keep their sign and get scale byte 0
    z = np.zeros(32)
    z[3] = -0.0
    c, s = oracle.mxfp8_block(z)
    assert s == 0 and c[3] == 0x80 and (np.delete(c, 3) == 0).all()
    # a tiny maximum: the scale stops at 2^-127
    c, s = oracle.mxfp8_block(np.full(32, 2.0 ** -130))
    assert s == 0 and oracle.e4m3_value(int(c[0])) * 2.0 ** -127 == 2.0 ** -130


def test_mxfp8_block_non_finite_elements_are_nan():
    """E4M3 has no infinity: NaN and +-inf elements get the NaN code 0x7F, and the block
    scale and the other codes are those of the finite elements alone."""
    rng = np.random.default_rng(77)
    v = rng.standard_normal(32) * 5.0
    w = v.copy()
    w[[2, 9, 30]] = [np.nan, np.inf, -np.inf]
    c, s = oracle.mxfp8_block(w)
    assert (c[[2, 9, 30]] == 0x7F).all() and all(math.isnan(oracle.e4m3_value(int(x))) for x in c[[2, 9, 30]])
    finite = np.delete(np.arange(32), [2, 9, 30])
    bc, bs = _brute_block(np.where(np.isfinite(w), w, 0.0))
    assert s == bs and np.array_equal(c[finite], bc[finite])
    # a block of nothing but non-finite values: scale byte 0, every code NaN
    c, s = oracle.mxfp8_block(np.full(32, np.inf))
    assert s == 0 and (c == 0x7F).all()


@pytest.mark.parametrize("seed", range(4))
def test_mxfp8_quantisation_is_idempotent(seed):
    rng = np.random.default_rng(100 + seed)
    v = rng.standard_normal(32) * 3.0
    c, s = oracle.mxfp8_block(v)
    deq = np.array([oracle.e4m3_value(int(x)) for x in c]) * 2.0 ** (s - 127)
    c2, s2 = oracle.mxfp8_block(deq)
    assert s2 == s and np.array_equal(c2, c)


def _mxfp8_values(v):
    out = np.empty(v.size)
    for b in range(0, v.size, 32):
        c, s = oracle.mxfp8_block(v[b:b + 32])
        out[b:b + 32] = [oracle.e4m3_value(int(x)) * 2.0 ** (s - 127) for x in c]
    return out


def test_mxfp8_expert_is_the_bf16_expert_on_quantised_inputs():
    """Gate/up on an h that MXFP8 represents exactly give the same a in both modes; y in
    MXFP8 mode is the dequantised down matrix applied to the quantised a (numpy)."""
    L, F = 64, 96
    rec = synth.expert_blob(31, L, F, 1)
    rng = np.random.default_rng(5)
    h_exact = _mxfp8_values(rng.standard_normal(L))
    h = f64_to_bf16_bits(h_exact)
    assert np.array_equal(bf16_bits_to_f64(h), h_exact)  # 4 significant bits fit bf16
    a_b, _ = oracle.expert(h, rec, L, F, act_format=oracle.ACT_BF16)
    a_m, y_m = oracle.expert(h, rec, L, F, act_format=oracle.ACT_MXFP8)
    assert np.array_equal(a_b, a_m)
    (_, _), (_, _), (dc, ds) = split_record(rec, L, F)
    Wd = np_dequant(dc, ds, L, F).astype(np.float64)
    y = (Wd @ _mxfp8_values(bf16_bits_to_f64(a_m))).astype(np.float32)
    assert np.array_equal(y_m, y)


def test_mxfp8_layer_differs_from_bf16_by_the_quantisation():
    """The MXFP8 mode changes the layer output by about the E4M3 rounding (3 mantissa
    bits), far more than the bf16 mode's tolerance and far less than the output."""
    T, d, L, F, E, k = 4, 64, 64, 96, 8, 2
    x = synth.normal_bf16(41, 1, 1.0, (T, d))
    Wr = synth.normal_bf16(41, 2, 0.02, (E, d))
    Wd = synth.normal_bf16(41, 3, 0.02, (L, d))
    Wu = synth.normal_bf16(41, 4, 0.02, (d, L))
    blob = synth.expert_blob(41, L, F, E)
    rb = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F)
    rm = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F, act_format=oracle.ACT_MXFP8)
    assert np.array_equal(rb["idx"], rm["idx"]) and np.array_equal(rb["h"], rm["h"])
    ob, om = bf16_bits_to_f64(rb["out"]), bf16_bits_to_f64(rm["out"])
    rel = np.linalg.norm(om - ob) / np.linalg.norm(ob)
    assert 3e-3 < rel < 0.1
