"""The seeded input generators, checked against their published definitions and the
distributions they are meant to draw, and bench.py's refusal of several GPUs.

Every input of the parity tests and of the benchmark comes from synth/, so a generator
that drifted (a wrong constant, a biased transform, a slice that depends on where the
generation started) would change every workload silently; these tests fix it.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest
from scipy import stats

import synth

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_splitmix64_published_sequence_from_state_zero():
    # Seed 0, stream 0 starts the counter at state 0 (the stream base mixes 0 to 0),
    # so the draws are splitmix64's own outputs from state 0 (Steele, Lea and Flood,
    # OOPSLA 2014): the first four are the widely printed reference values.
    L = synth.lib()
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert [L.synth_draw(0, 0, i) for i in range(4)] == want


def test_streams_and_seeds_give_different_draws():
    L = synth.lib()
    a = [L.synth_draw(1, 1, i) for i in range(64)]
    b = [L.synth_draw(1, 2, i) for i in range(64)]
    c = [L.synth_draw(2, 1, i) for i in range(64)]
    assert len(set(a)) == 64 and not set(a) & set(b) and not set(a) & set(c)


def test_draw_bits_are_balanced():
    # each of the 64 output bits is set in about half of 20,000 draws (4.5 sigma band)
    L = synth.lib()
    n = 20000
    d = np.array([L.synth_draw(7, 3, i) for i in range(n)], dtype=np.uint64)
    ones = np.array([int(((d >> np.uint64(b)) & np.uint64(1)).sum()) for b in range(64)])
    assert np.all(np.abs(ones - n / 2) < 4.5 * math.sqrt(n) / 2)


def test_normals_follow_the_standard_normal():
    L = synth.lib()
    v = np.array([L.synth_normal(11, 5, i) for i in range(20000)])
    assert stats.kstest(v, "norm").pvalue > 1e-3
    assert abs(v.mean()) < 4.5 / math.sqrt(v.size)


def test_bf16_normals_scale_and_round():
    # std 0.02 as the dense weights use: sample moments, and every value is the
    # round-to-nearest-even bf16 of its fp32 draw
    n = 1 << 20
    bits = synth.normal_bf16(13, 2, 0.02, n)
    f = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f.mean()) < 4.5 * 0.02 / math.sqrt(n)
    assert abs(f.std() / 0.02 - 1.0) < 0.005
    L = synth.lib()
    for i in range(0, 64):
        x = np.float32(0.02 * L.synth_normal(13, 2, i))
        u = int(np.array([x]).view(np.uint32)[0])
        rne = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        assert int(bits[i]) == rne


def test_slices_do_not_depend_on_where_generation_starts():
    full = synth.normal_bf16(17, 4, 1.0, 300)
    part = synth.normal_bf16(17, 4, 1.0, 100, first=150)
    assert np.array_equal(full[150:250], part)


def test_permutation_is_a_seeded_permutation():
    p = synth.permutation(19, 7, 896)
    assert np.array_equal(np.sort(p), np.arange(896))
    assert np.array_equal(p, synth.permutation(19, 7, 896))
    assert not np.array_equal(p, synth.permutation(20, 7, 896))
    assert not np.array_equal(p, np.arange(896))


def test_categorical_is_uniform():
    m, n = 4, 40000
    c = synth.categorical(23, 8, n, m)
    assert c.min() >= 0 and c.max() < m
    assert stats.chisquare(np.bincount(c, minlength=m)).pvalue > 1e-3


def test_expert_blob_codes_and_scales():
    # one tiny record: code nibbles uniform over the 16 E2M1 codes, scale bytes within
    # the requested exponent range and covering it
    L, F = 128, 64
    rec = synth.expert_blob(29, L, F, 2, scale_lo=120, scale_hi=130)
    assert rec.size == 2 * synth.expert_record_bytes(L, F)
    per = synth.expert_record_bytes(L, F) // 3
    codes, scales = [], []
    for e in range(2):
        for m in range(3):
            base = e * 3 * per + m * per
            codes.append(rec[base:base + L * F // 2])
            scales.append(rec[base + L * F // 2:base + per])
    cb = np.concatenate(codes)
    nib = np.concatenate([cb & 15, cb >> 4])
    assert stats.chisquare(np.bincount(nib, minlength=16)).pvalue > 1e-3
    sc = np.concatenate(scales)
    assert sc.min() == 120 and sc.max() == 130


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=REPO)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["decode1", "prefill4k"])
def test_bench_configs_have_the_k3_shapes(name):
    c = synth.CONFIGS[name]
    assert (c.d, c.L, c.F, c.E, c.k) == (7168, 3584, 3072, 896, 16)
    assert c.record_bytes == 17547264
