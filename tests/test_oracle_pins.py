"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test compares the oracle with something other than itself: values the
pages print (fixtures under tests/golden/), closed forms, invariants, special
cases that reduce to a library routine, and brute force or exact rational
arithmetic on tiny inputs.  No expected value here comes from the GPU path.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from _util import (GOLDEN, bf16_bits_to_f64, bf16_fraction, e2m1_table, f64_to_bf16_bits,
                   fraction_to_f32, np_dequant, rel_l2, split_record)


# ---------------------------------------------------------------- format pins

def test_e2m1_table_matches_golden():
    want = e2m1_table()
    got = np.array([oracle.e2m1(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # code 8 is -0


def test_mxfp4_value_exhaustive_16x256():
    """Every (code, e8m0) pair: E2M1(code) * 2^(s-127) rounded to fp32; s = 255 is NaN."""
    lut = e2m1_table()
    for s in range(256):
        for c in range(16):
            got = oracle.mxfp4_value(c, s)
            if s == 255:
                assert math.isnan(got)
                continue
            want = float(np.float32(math.ldexp(lut[c], s - 127)))  # exact, or inf past fp32 range
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, s, got, want)


def _read_rows_fixture():
    rows = {}
    with open(os.path.join(GOLDEN, "mxfp4_rows.txt")) as fh:
        for line in fh:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            r = int(p[1])
            rows.setdefault(r, {})
            if p[0] == "codes":
                rows[r]["codes"] = bytes(int(v, 16) for v in p[2:])
            elif p[0] == "scales":
                rows[r]["scales"] = bytes(int(v) for v in p[2:])
            elif p[0] == "expect":
                rows[r]["expect"] = [float.fromhex(v) if v.startswith(("0x", "-0x")) else float(v)
                                     for v in p[2:]]
    return rows


def test_dequant_layout_golden_rows():
    rows = _read_rows_fixture()
    n = len(rows)
    codes = np.frombuffer(b"".join(rows[r]["codes"] for r in range(n)), dtype=np.uint8).copy()
    scales = np.frombuffer(b"".join(rows[r]["scales"] for r in range(n)), dtype=np.uint8).copy()
    got = oracle.dequant_matrix(codes, scales, n, 64)
    for r in range(n):
        want = np.array(rows[r]["expect"], dtype=np.float32)
        assert want.size == 64
        same = (got[r] == want) | (np.isnan(got[r]) & np.isnan(want))
        assert same.all(), (r, np.nonzero(~same))
        assert np.array_equal(np.signbit(got[r][~np.isnan(want)]), np.signbit(want[~np.isnan(want)]))


def test_dequant_matches_numpy_reading_of_layout():
    """A random record dequantised by the oracle equals numpy's reading of the same layout."""
    L, F = 128, 96
    rec = synth.expert_blob(7, L, F, 1, scale_lo=0, scale_hi=255)
    for (codes, scales), (rows, cols) in zip(split_record(rec, L, F), [(F, L), (F, L), (L, F)]):
        got = oracle.dequant_matrix(np.ascontiguousarray(codes), np.ascontiguousarray(scales), rows, cols)
        want = np_dequant(codes, scales, rows, cols)
        same = (got == want) | (np.isnan(got) & np.isnan(want))
        assert same.all()


def test_expert_bytes_closed_forms_and_page_cross_checks():
    with open(os.path.join(GOLDEN, "expert_sizes.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                L, F, b = map(int, line.split())
                assert oracle.expert_bytes(L, F) == b
                assert synth.expert_record_bytes(L, F) == b
    per_expert = 3 * 3584 * 3072
    assert per_expert == 33_030_144
    assert per_expert * 0.53125 == 17_547_264
    # 896 experts x 92 routed layers = 82,432 experts; 2722.7B params; ~1.447 TB
    assert 896 * 92 == 82_432
    assert round(82_432 * per_expert / 1e9, 1) == 2722.7
    assert round(82_432 * 17_547_264 / 1e12, 3) == 1.446  # the post rounds to "1.447TB"
    # 16 active experts x 92 layers ~ 26 GB per token
    assert round(16 * 92 * 17_547_264 / 1e9) == 26
    # 4.25 bits per weight
    assert 17_547_264 * 8 / per_expert == 4.25


# ------------------------------------------------------------- rounding pins

@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie, even stays
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie, rounds to even mantissa
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie
    (2.0 ** -133, 0x0001),                     # smallest bf16 subnormal
    (2.0 ** -134, 0x0000),                     # tie to even -> 0
    (1.5 * 2.0 ** -134, 0x0001),
    (-(2.0 ** -126), 0x8080),
    (3.4e38, 0x7F80),                          # past (2 - 2^-8) * 2^127 -> inf
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite bf16
    (-0.0, 0x8000),
    (float("nan"), 0x7FC0),
    (-float("inf"), 0xFF80),
])
def test_bf16_rounding_closed_forms(v, bits):
    assert oracle.bf16_from_f64(v) == bits


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for g in [0.1, 1.0, 2.5, 10.0, 30.0]:
        assert abs(oracle.silu(g) - oracle.silu(-g) - g) <= 1e-15 * max(1.0, g)
    assert abs(oracle.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15  # sigmoid(ln 3) = 3/4
    assert oracle.silu(-1000.0) == 0.0 and oracle.silu(1000.0) == 1000.0


# ------------------------------------------------------- exact router logits

def _rand_bf16(rng, n, lo_exp=1, hi_exp=254):
    sign = rng.integers(0, 2, n) << 15
    ex = rng.integers(lo_exp, hi_exp + 1, n) << 7
    fr = rng.integers(0, 128, n)
    return (sign | ex | fr).astype(np.uint16)


def _exact_dot_frac(a, b):
    return sum((bf16_fraction(int(x)) * bf16_fraction(int(y)) for x, y in zip(a, b)), Fraction(0))


@pytest.mark.parametrize("case", range(6))
def test_exact_dot_vs_fractions_wide_exponents(case):
    rng = np.random.default_rng(100 + case)
    n = [1, 7, 64, 200, 33, 128][case]
    lo, hi = [(1, 254), (100, 160), (0, 254), (110, 140), (1, 20), (235, 254)][case]
    a = _rand_bf16(rng, n, lo, hi)
    b = _rand_bf16(rng, n, lo, hi)
    want = fraction_to_f32(_exact_dot_frac(a, b))
    got = oracle.dot_bf16_exact(a, b)
    assert got == want or (math.isinf(want) and got == want), (got, want)


def test_exact_dot_vs_fractions_k3_like():
    """Router-like data: x ~ N(0,1), w ~ N(0,0.02), d = 7168."""
    x = synth.normal_bf16(11, 1, 1.0, 7168)
    for e in range(4):
        w = synth.normal_bf16(11, 2, 0.02, 7168, first=e * 7168)
        assert oracle.dot_bf16_exact(x, w) == fraction_to_f32(_exact_dot_frac(x, w))


def _bf(v: float) -> int:
    """bf16 bits of a value exactly representable in bf16."""
    b = int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)
    assert bf16_fraction(b) == Fraction(v)
    return b


def test_exact_dot_ties_and_sticky_bits():
    one, tiny = _bf(1.0), _bf(2.0 ** -12)
    # 1 + 2^-24 is halfway between 1 and 1 + 2^-23: ties to even -> 1
    assert oracle.dot_bf16_exact(np.array([one, tiny], np.uint16), np.array([one, tiny], np.uint16)) == 1.0
    # the same plus 2^-120 must round up: the sticky bit sits ~100 bits below
    far = _bf(2.0 ** -60)
    got = oracle.dot_bf16_exact(np.array([one, tiny, far], np.uint16), np.array([one, tiny, far], np.uint16))
    assert got == 1.0 + 2.0 ** -23
    # and minus 2^-120 must round down
    nfar = _bf(-(2.0 ** -60))
    got = oracle.dot_bf16_exact(np.array([one, tiny, nfar], np.uint16), np.array([one, tiny, far], np.uint16))
    assert got == 1.0
    # exact cancellation, then a tiny remainder survives exactly
    a = np.array([_bf(3.0), _bf(-3.0), _bf(2.0 ** -70)], np.uint16)
    b = np.array([_bf(2.0 ** 60), _bf(2.0 ** 60), _bf(2.0 ** -70)], np.uint16)
    assert oracle.dot_bf16_exact(a, b) == 2.0 ** -140
    # subnormal fp32 result
    a = np.array([_bf(2.0 ** -75), _bf(2.0 ** -76)], np.uint16)
    b = np.array([_bf(2.0 ** -75), _bf(2.0 ** -76)], np.uint16)
    assert oracle.dot_bf16_exact(a, b) == fraction_to_f32(Fraction(2) ** -150 + Fraction(2) ** -152)
    # negative result, and zero
    assert oracle.dot_bf16_exact(np.array([_bf(-2.0)], np.uint16), np.array([_bf(3.0)], np.uint16)) == -6.0
    z = oracle.dot_bf16_exact(np.array([_bf(2.0), _bf(-2.0)], np.uint16), np.array([_bf(1.0), _bf(1.0)], np.uint16))
    assert z == 0.0 and math.copysign(1.0, z) == 1.0
    # overflow to inf, and IEEE specials
    big = _bf(2.0 ** 127)
    assert oracle.dot_bf16_exact(np.array([big, big], np.uint16), np.array([_bf(2.0), _bf(2.0)], np.uint16)) == math.inf
    inf, nan = 0x7F80, 0x7FC0
    assert oracle.dot_bf16_exact(np.array([inf, one], np.uint16), np.array([one, one], np.uint16)) == math.inf
    assert math.isnan(oracle.dot_bf16_exact(np.array([inf], np.uint16), np.array([0], np.uint16)))
    assert math.isnan(oracle.dot_bf16_exact(np.array([nan], np.uint16), np.array([one], np.uint16)))
    assert math.isnan(oracle.dot_bf16_exact(np.array([inf, inf], np.uint16), np.array([one, 0xBF80], np.uint16)))


def _router_one(a, b):
    """The oracle's router logit of one token against one router row."""
    return float(oracle.router_logits(np.ascontiguousarray(a, np.uint16)[None, :],
                                      np.ascontiguousarray(b, np.uint16)[None, :])[0, 0])


@pytest.mark.parametrize("case", range(6))
def test_router_logit_vs_fractions_wide_exponents(case):
    """The router's logit (fp64 sum with an error bound, exact accumulator when the bound
    cannot decide) is the correctly rounded exact dot, across the whole bf16 range."""
    rng = np.random.default_rng(200 + case)
    n = [1, 7, 64, 200, 33, 128][case]
    lo, hi = [(1, 254), (100, 160), (0, 254), (110, 140), (1, 20), (235, 254)][case]
    for _ in range(20):
        a = _rand_bf16(rng, n, lo, hi)
        b = _rand_bf16(rng, n, lo, hi)
        want = fraction_to_f32(_exact_dot_frac(a, b))
        assert _router_one(a, b) == want


def test_router_logit_decided_exactly_near_rounding_boundaries():
    """Sums within a few fp64 ulps of an fp32 rounding midpoint, where a plain fp64 sum
    rounded to fp32 gives the wrong value: the bound must send them to the exact path."""
    one, tiny, far, nfar = _bf(1.0), _bf(2.0 ** -12), _bf(2.0 ** -60), _bf(-(2.0 ** -60))
    # 1 + 2^-24 + 2^-120: fp64 keeps 1 + 2^-24, a tie that rounds to 1; exactly it rounds up
    assert _router_one([one, tiny, far], [one, tiny, far]) == 1.0 + 2.0 ** -23
    assert _router_one([one, tiny, nfar], [one, tiny, far]) == 1.0
    assert _router_one([one, tiny], [one, tiny]) == 1.0
    # exact cancellation: +0, and a tiny survivor
    z = _router_one([_bf(2.0), _bf(-2.0)], [_bf(1.0), _bf(1.0)])
    assert z == 0.0 and math.copysign(1.0, z) == 1.0
    assert _router_one([_bf(3.0), _bf(-3.0), _bf(2.0 ** -70)], [_bf(2.0 ** 60), _bf(2.0 ** 60), _bf(2.0 ** -70)]) \
        == 2.0 ** -140
    # a negative sum just below zero rounds to -0 in fp32; just above, to +0
    s = _router_one([_bf(2.0 ** -80)], [_bf(-(2.0 ** -80))])
    assert s == 0.0 and math.copysign(1.0, s) == -1.0
    # all products zero (signed zeros included): +0
    s = _router_one([0x8000, 0x0000], [0x3F80, 0xBF80])
    assert s == 0.0 and math.copysign(1.0, s) == 1.0
    # specials go to the exact path's IEEE rules
    inf, nan = 0x7F80, 0x7FC0
    assert _router_one([inf, one], [one, one]) == math.inf
    assert math.isnan(_router_one([inf], [0]))
    assert math.isnan(_router_one([nan], [one]))
    assert _router_one([_bf(2.0 ** 127), _bf(2.0 ** 127)], [_bf(2.0), _bf(2.0)]) == math.inf
    # random sums planted on fp32 midpoints, then nudged by one product far below
    rng = np.random.default_rng(7)
    for _ in range(200):
        m = int(rng.integers(1 << 7, 1 << 8))
        e = int(rng.integers(-20, 20))
        # m * 2^e * (1 + 2^-8 + ...) : choose a, b so that the exact sum is v + half an fp32 ulp of v
        v = Fraction(m) * Fraction(2) ** e
        vf = float(v)
        ulp_half = Fraction(2) ** (math.frexp(vf)[1] - 25)
        hb = fraction_to_f32(ulp_half)
        nudge = int(rng.integers(-1, 2))
        a = [_bf(vf), _bf(hb), _bf(2.0 ** -70) if nudge else 0]
        b = [one, one, _bf(float(nudge) * 2.0 ** -60) if nudge else 0]
        want = fraction_to_f32(_exact_dot_frac(np.array(a, np.uint16), np.array(b, np.uint16)))
        assert _router_one(a, b) == want


def test_router_logits_equal_exact_dot_k3_router():
    """Every logit of two K3-shaped tokens against the whole 896 x 7168 router equals the
    exact accumulator's value bit for bit."""
    c = synth.CONFIGS["decode1"]
    x = synth.make_tokens(c, T=2)
    W = synth.make_dense(c)["router_w"]
    got = oracle.router_logits(x, W)
    for t in range(2):
        for e in range(c.E):
            assert got[t, e] == oracle.dot_bf16_exact(x[t], W[e]), (t, e)


def test_router_bias_is_one_fp32_add():
    c = synth.CONFIGS["tiny"]
    x = synth.make_tokens(c)
    W = synth.make_dense(c)["router_w"]
    bias = np.linspace(-3, 3, c.E).astype(np.float32)
    l0 = oracle.router_logits(x, W)
    l1 = oracle.router_logits(x, W, bias)
    assert np.array_equal(l1, (l0 + bias[None, :]).astype(np.float32))
    bias2 = np.arange(c.T * c.E, dtype=np.float32).reshape(c.T, c.E) / 7
    l2 = oracle.router_logits(x, W, bias2)
    assert np.array_equal(l2, (l0 + bias2).astype(np.float32))
    # no bias: every logit equals the fp64 dot rounded to fp32 (exact here: spread < 53 bits)
    want = (bf16_bits_to_f64(x) @ bf16_bits_to_f64(W).T).astype(np.float32)
    assert np.array_equal(l0, want)


# --------------------------------------------------------------- selection

def _ranks_before(va, ia, vb, ib):
    if math.isnan(va) != math.isnan(vb):
        return math.isnan(vb)
    if not math.isnan(va) and va != vb:
        return va > vb
    return ia < ib


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_select_brute_force_all_subsets(k):
    """The top-k set is the unique subset whose members all rank before all non-members."""
    rng = np.random.default_rng(k)
    E, T = 8, 200
    pool = np.array([-1.0, 0.0, -0.0, 1.0, 2.0, np.nan, -np.inf, np.inf, 0.5], dtype=np.float32)
    logits = pool[rng.integers(0, pool.size, (T, E))]
    logits[:20] = rng.standard_normal((20, E)).astype(np.float32)
    idx, w = oracle.select(logits, k)
    for t in range(T):
        l = logits[t]
        winners = []
        for S in itertools.combinations(range(E), k):
            rest = [j for j in range(E) if j not in S]
            if all(_ranks_before(l[i], i, l[j], j) for i in S for j in rest):
                winners.append(S)
        assert len(winners) == 1
        assert tuple(idx[t]) == winners[0]


def test_select_weights_softmax_and_sum():
    c = synth.CONFIGS["tiny"]
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((64, c.E)) * 2).astype(np.float32)
    for k in (1, 2, 5):
        idx, w = oracle.select(logits, k)
        sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
        p = np.exp(sel - sel.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.allclose(w, p, rtol=1e-6, atol=0)
        assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
        _, w_all = oracle.select(logits, k, renormalize=False)
        q = np.exp(logits - logits.max(1, keepdims=True)).astype(np.float64)
        q /= q.sum(1, keepdims=True)
        assert np.allclose(w_all, np.take_along_axis(q, idx, 1), rtol=1e-6, atol=0)


# --------------------------------------------------------------- permutation

def test_permute_equals_stable_argsort_and_invariants():
    rng = np.random.default_rng(5)
    E, k, T = 37, 5, 300
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.permute(idx, E)
    flat = idx.ravel()
    assert np.array_equal(perm, np.argsort(flat, kind="stable").astype(np.int32))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(T * k))


def test_routing_invariants_tiny_and_k3_router():
    for name, T in (("tiny", None), ("decode64", 16)):
        c = synth.CONFIGS[name]
        x = synth.make_tokens(c, T=T)
        W = synth.make_dense(c)["router_w"] if name == "tiny" else synth.normal_bf16(c.layer_seed, synth.S_ROUTER,
                                                                                      0.02, (c.E, c.d))
        idx, w = oracle.select(oracle.router_logits(x, W), c.k)
        for t in range(idx.shape[0]):
            assert len(set(idx[t].tolist())) == c.k                      # k distinct experts
            assert list(idx[t]) == sorted(idx[t])                         # ascending ids
        counts, _, _ = oracle.permute(idx, c.E)
        assert counts.sum() == idx.shape[0] * c.k                         # routed exactly k times
        assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ combine

def test_combine_identity_expert_equals_weight_sum_times_h():
    """With every expert the identity (y := h), z = bf16((sum_j w_j) h), and sum_j w_j = 1."""
    rng = np.random.default_rng(9)
    T, k, L = 32, 4, 64
    h = f64_to_bf16_bits(rng.standard_normal((T, L)))
    _, w = oracle.select(rng.standard_normal((T, 11)).astype(np.float32), k)
    y = np.repeat(bf16_bits_to_f64(h).astype(np.float32), k, axis=0)
    z = oracle.combine(y, w)
    want = f64_to_bf16_bits(w.astype(np.float64).sum(1, keepdims=True) * bf16_bits_to_f64(h))
    assert np.array_equal(z, want)
    # and that is h itself to within one bf16 ulp
    assert np.max(np.abs(z.astype(np.int64) - h.astype(np.int64))) <= 1


def test_combine_one_hot_and_pow2_scaling():
    rng = np.random.default_rng(10)
    T, k, L = 8, 3, 32
    y = rng.standard_normal((T * k, L)).astype(np.float32)
    for j in range(k):
        w = np.zeros((T, k), np.float32)
        w[:, j] = 1.0
        z = oracle.combine(y, w)
        assert np.array_equal(z, f64_to_bf16_bits(y.reshape(T, k, L)[:, j, :].astype(np.float64)))
    w = rng.random((T, k)).astype(np.float32)
    z1 = bf16_bits_to_f64(oracle.combine(y, w))
    z8 = bf16_bits_to_f64(oracle.combine(y * np.float32(8), w))
    assert np.array_equal(z8, 8 * z1)


# --------------------------------------------------------------- dense parts

def test_linear_matches_numpy_matmul():
    rng = np.random.default_rng(12)
    a = f64_to_bf16_bits(rng.standard_normal((5, 96)))
    W = f64_to_bf16_bits(0.02 * rng.standard_normal((40, 96)))
    got = oracle.linear_bf16(a, W)
    want = f64_to_bf16_bits(bf16_bits_to_f64(a) @ bf16_bits_to_f64(W).T)
    assert np.array_equal(got, want)


# ----------------------------------------------------- layer special cases

def _np_glu_expert(h_bits, record, L, F):
    (gc, gs), (uc, us), (dc, ds) = split_record(record, L, F)
    Wg = np_dequant(gc, gs, F, L).astype(np.float64)
    Wu = np_dequant(uc, us, F, L).astype(np.float64)
    Wd = np_dequant(dc, ds, L, F).astype(np.float64)
    h = bf16_bits_to_f64(h_bits)
    g = (Wg @ h).astype(np.float32).astype(np.float64)
    u = (Wu @ h).astype(np.float32).astype(np.float64)
    a = f64_to_bf16_bits(g / (1.0 + np.exp(-g)) * u)
    y = (Wd @ bf16_bits_to_f64(a)).astype(np.float32)
    return a, y


def _np_dequant_exact(codes, scales, rows, cols):
    """The weights' exact values in fp64 from the golden table: E2M1 * 2^(s-127), NaN for s = 255."""
    lut = e2m1_table()
    c = codes.reshape(rows, cols // 2)
    nib = np.empty((rows, cols), dtype=np.int64)
    nib[:, 0::2] = c & 15
    nib[:, 1::2] = c >> 4
    s = np.repeat(scales.reshape(rows, cols // 32).astype(np.int64), 32, axis=1)
    w = np.ldexp(lut[nib], s - 127)
    w[s == 255] = np.nan
    return w


def _np_glu_expert_exact(h_bits, record, L, F):
    (gc, gs), (uc, us), (dc, ds) = split_record(record, L, F)
    h = bf16_bits_to_f64(h_bits)
    with np.errstate(all="ignore"):
        g = (_np_dequant_exact(gc, gs, F, L) @ h).astype(np.float32).astype(np.float64)
        u = (_np_dequant_exact(uc, us, F, L) @ h).astype(np.float32).astype(np.float64)
        a = f64_to_bf16_bits(g / (1.0 + np.exp(-g)) * u)
        y = (_np_dequant_exact(dc, ds, L, F) @ bf16_bits_to_f64(a)).astype(np.float32)
    return a, y


def _same_bits_or_nan(a, b):
    a, b = np.asarray(a), np.asarray(b)
    fa = a.astype(np.float64) if a.dtype != np.uint16 else bf16_bits_to_f64(a)
    fb = b.astype(np.float64) if b.dtype != np.uint16 else bf16_bits_to_f64(b)
    return bool(((fa == fb) & (np.signbit(fa) == np.signbit(fb)) | (np.isnan(fa) & np.isnan(fb))).all())


def test_expert_extreme_scales_use_exact_weight_values():
    """Records with e8m0 scales at both ends of the range (0 = 2^-127, 1-20, 235-254) and
    NaN blocks (255): the oracle's expert equals an fp64 numpy GLU on the weights' exact
    values, NaN included.  With h tiny enough, scales 253-254 give finite products although
    their large weights lie past the fp32 range (no fp32 rounding of weights happens)."""
    L, F = 64, 96
    nc, ns = F * L // 2, F * L // 32
    mat = nc + ns
    cases = [  # (gate/up scale range, down scale range, h exponent, 255 blocks in (matrix, block index))
        ((0, 0), (120, 130), 100, []),
        ((1, 20), (1, 20), 100, []),
        ((235, 254), (120, 130), -100, []),
        ((60, 80), (235, 254), 0, []),
        ((120, 130), (120, 130), 0, [(0, 5)]),
        ((120, 130), (120, 130), 0, [(2, 7)]),
        ((0, 254), (0, 254), 0, []),
    ]
    rng = np.random.default_rng(31)
    saw_big = False
    for n, (gu, dn, hexp, nan_blocks) in enumerate(cases):
        rec = synth.expert_blob(500 + n, L, F, 1).copy()
        for m, (lo, hi) in enumerate((gu, gu, dn)):
            rec[m * mat + nc:(m + 1) * mat] = rng.integers(lo, hi + 1, ns)
        for m, b in nan_blocks:
            rec[m * mat + nc + b] = 255
        h = f64_to_bf16_bits(rng.standard_normal(L) * 2.0 ** hexp)
        a_o, y_o = oracle.expert(h, rec, L, F)
        a_n, y_n = _np_glu_expert_exact(h, rec, L, F)
        assert _same_bits_or_nan(a_o, a_n), n
        assert _same_bits_or_nan(y_o, y_n), n
        if gu[1] == 254 and hexp < 0:
            saw_big = True
            assert np.isfinite(y_o).all() and np.isfinite(bf16_bits_to_f64(a_o)).all()
            # the fp32-rounded weights would have been infinite
            assert np.isinf(np_dequant(*split_record(rec, L, F)[0], F, L)).any()
        if nan_blocks:
            m, b = nan_blocks[0]
            if m == 0:  # a gate row holding NaN makes that a NaN and so every y NaN
                assert np.isnan(y_o).all()
            else:       # a down row holding NaN makes that y NaN only
                row = b // (F // 32)
                assert np.isnan(y_o[row]) and np.isfinite(np.delete(y_o, row)).all()
    assert saw_big


def _tiny_layer(E, seed=21, d=64, L=64, F=96, T=6):
    rng_seed = seed
    x = synth.normal_bf16(rng_seed, 1, 1.0, (T, d))
    Wr = synth.normal_bf16(rng_seed, 2, 0.02, (E, d))
    Wd = synth.normal_bf16(rng_seed, 3, 0.02, (L, d))
    Wu = synth.normal_bf16(rng_seed, 4, 0.02, (d, L))
    blob = synth.expert_blob(rng_seed, L, F, E)
    return x, Wr, Wd, Wu, blob, d, L, F, T


def test_single_expert_layer_is_a_dense_glu_mlp():
    """E = 1, k = 1: routing is trivial (weight 1) and the layer is a dense GLU MLP."""
    x, Wr, Wd, Wu, blob, d, L, F, T = _tiny_layer(E=1)
    r = oracle.layer_forward(x, Wr, Wd, Wu, blob, 1, L, F)
    assert (r["idx"] == 0).all() and (r["w"] == 1.0).all()
    h = f64_to_bf16_bits(bf16_bits_to_f64(x) @ bf16_bits_to_f64(Wd).T)
    assert np.array_equal(r["h"], h)
    for t in range(T):
        a, y = _np_glu_expert(h[t], blob, L, F)
        a_o, y_o = oracle.expert(h[t], blob, L, F)
        assert np.array_equal(a_o, a) and np.array_equal(y_o, y)
        z = f64_to_bf16_bits(y.astype(np.float64))
        assert np.array_equal(r["z"][t], z)
        out = f64_to_bf16_bits(bf16_bits_to_f64(Wu) @ bf16_bits_to_f64(z))
        assert np.array_equal(r["out"][t], out)


def test_all_experts_selected_is_a_softmax_mixture():
    """k = E: every expert is used with the softmax of all logits as its weight."""
    E = 4
    x, Wr, Wd, Wu, blob, d, L, F, T = _tiny_layer(E=E, seed=22)
    r = oracle.layer_forward(x, Wr, Wd, Wu, blob, E, L, F)
    rec = synth.expert_record_bytes(L, F)
    logits = (bf16_bits_to_f64(x) @ bf16_bits_to_f64(Wr).T).astype(np.float32)
    assert np.array_equal(r["logits"], logits)
    p = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(r["w"], p, rtol=1e-6, atol=0)
    h = f64_to_bf16_bits(bf16_bits_to_f64(x) @ bf16_bits_to_f64(Wd).T)
    for t in range(T):
        ys = [_np_glu_expert(h[t], blob[e * rec:(e + 1) * rec], L, F)[1] for e in range(E)]
        z = f64_to_bf16_bits(sum(float(r["w"][t, e]) * ys[e].astype(np.float64) for e in range(E)))
        assert np.array_equal(r["z"][t], z)
        out = f64_to_bf16_bits(bf16_bits_to_f64(Wu) @ bf16_bits_to_f64(z))
        assert rel_l2(bf16_bits_to_f64(r["out"][t]), bf16_bits_to_f64(out)) < 1e-6


def test_expert_relabelling_leaves_outputs_unchanged():
    """Renaming experts (router rows and blob records permuted together) changes nothing
    but the reported ids: catches any mix-up between an expert id and its record."""
    E, k = 8, 3
    x, Wr, Wd, Wu, blob, d, L, F, T = _tiny_layer(E=E, seed=23, T=10)
    rec = synth.expert_record_bytes(L, F)
    pi = np.array([5, 2, 7, 0, 3, 6, 1, 4])
    Wr2 = np.ascontiguousarray(Wr[pi])
    blob2 = np.concatenate([blob[p * rec:(p + 1) * rec] for p in pi])
    r1 = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F)
    r2 = oracle.layer_forward(x, Wr2, Wd, Wu, blob2, k, L, F)
    for t in range(T):
        assert sorted(pi[r2["idx"][t]].tolist()) == r1["idx"][t].tolist()
    # only the order of the fp64 combine sum changes, so at most a rare bf16 tie flips
    assert rel_l2(bf16_bits_to_f64(r2["out"]), bf16_bits_to_f64(r1["out"])) < 1e-5


def test_token_subset_rows_equal_full_run_rows():
    c = synth.CONFIGS["tiny"]
    Ly = synth.make_layer(c)
    full = oracle.layer_forward(Ly["x"], Ly["router_w"], Ly["latent_down"], Ly["latent_up"], Ly["blob"], c.k, c.L, c.F)
    sub = [13, 2, 7]
    part = oracle.layer_forward(Ly["x"], Ly["router_w"], Ly["latent_down"], Ly["latent_up"], Ly["blob"], c.k, c.L,
                                c.F, tokens=sub)
    for key in ("out", "idx", "w", "logits", "h", "z"):
        assert np.array_equal(part[key], full[key][sub])


def test_situ_activation_rejected():
    c = synth.CONFIGS["tiny"]
    Ly = synth.make_layer(c)
    with pytest.raises(RuntimeError):
        oracle.layer_forward(Ly["x"], Ly["router_w"], Ly["latent_down"], Ly["latent_up"], Ly["blob"], c.k, c.L, c.F,
                             act=oracle.ACT_SITU)


# ------------------------------------------------------------ shared experts

def _zero_down(blob, L, F, E):
    """The records with their down matrices' codes set to zero (+0), scales kept."""
    out = blob.copy()
    rec = synth.expert_record_bytes(L, F)
    mat = F * L // 2 + F * L // 32
    for e in range(E):
        out[e * rec + 2 * mat:e * rec + 2 * mat + F * L // 2] = 0
    return out


def test_shared_experts_none_is_the_routed_layer():
    x, Wr, Wd, Wu, blob, d, L, F, T = _tiny_layer(E=6, seed=61)
    a = oracle.layer_forward(x, Wr, Wd, Wu, blob, 2, L, F)
    b = oracle.layer_forward(x, Wr, Wd, Wu, blob, 2, L, F, shared_blob=synth.expert_blob(62, d, 64, 2), num_shared=0,
                             d_ffn_shared=64)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_shared_experts_alone_are_dense_glu_mlps_on_x():
    """Routed experts whose down matrices are zero give z = 0, so out is the bf16 of the
    sum of the shared experts' outputs, each a dense GLU MLP on the full-width x."""
    E, k, F_s, S = 6, 2, 64, 2
    x, Wr, Wd, Wu, blob, d, L, F, T = _tiny_layer(E=E, seed=63)
    shared = synth.expert_blob(64, d, F_s, S)
    r = oracle.layer_forward(x, Wr, Wd, Wu, _zero_down(blob, L, F, E), k, L, F, shared_blob=shared, num_shared=S,
                             d_ffn_shared=F_s)
    assert (r["z"] == 0).all()
    srec = synth.expert_record_bytes(d, F_s)
    for t in range(T):
        ys = [_np_glu_expert(x[t], shared[s * srec:(s + 1) * srec], d, F_s)[1].astype(np.float64) for s in range(S)]
        assert np.array_equal(r["out"][t], f64_to_bf16_bits(ys[0] + ys[1]))


def test_shared_experts_with_zero_output_leave_the_layer():
    E, k, F_s = 6, 2, 64
    x, Wr, Wd, Wu, blob, d, L, F, T = _tiny_layer(E=E, seed=65)
    shared = _zero_down(synth.expert_blob(66, d, F_s, 2), d, F_s, 2)
    a = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F)
    b = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F, shared_blob=shared, num_shared=2, d_ffn_shared=F_s)
    assert np.array_equal(a["out"], b["out"])


# ------------------------------------------------- expert layout (cosine check)

def test_expert_cosine_detects_layout_mistakes():
    """The per-expert cosine check of the GPU tests catches layout mistakes: with gate and
    up swapped, the three matrices of a record mis-stacked by one, or the neighbouring
    record read, the oracle's own expert output moves far from the correct one, while the
    GPU tests require a cosine of at least 0.9999 (the layer's kimi-k3-mlx verification idea:
    a mis-stacked or transposed expert drives the similarity towards zero)."""
    from _util import cosine
    c = synth.CONFIGS["tiny"]
    lay = synth.make_layer(c)
    hl = oracle.linear_bf16(lay["x"], lay["latent_down"])
    rec = c.record_bytes
    mb = rec // 3  # gate, up and down have the same size at the tiny shape (L == F)
    for e in range(c.E):
        r = lay["blob"][e * rec:(e + 1) * rec]
        nxt = lay["blob"][((e + 1) % c.E) * rec:((e + 1) % c.E + 1) * rec]
        swapped = np.concatenate([r[mb:2 * mb], r[:mb], r[2 * mb:]])
        rotated = np.concatenate([r[mb:], r[:mb]])
        for t in range(2):
            _, y = oracle.expert(hl[t], r, c.L, c.F)
            assert cosine(y, oracle.expert(hl[t], r, c.L, c.F)[1]) == pytest.approx(1.0, abs=1e-12)
            assert cosine(y, oracle.expert(hl[t], swapped, c.L, c.F)[1]) < 0.95
            assert abs(cosine(y, oracle.expert(hl[t], rotated, c.L, c.F)[1])) < 0.6
            assert abs(cosine(y, oracle.expert(hl[t], nxt, c.L, c.F)[1])) < 0.6
