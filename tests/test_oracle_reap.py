"""Pins of the REAP pieces (kimi-k3-mlx digest, REAP section): the saliency sum
S_j |C| = sum over tokens of g_j ||e_j||_2 and pruning as a router bias of -inf with the
weights renormalised over the experts left."""
import numpy as np
import pytest

import oracle
import synth
from _util import bf16_bits_to_f64


def test_saliency_closed_forms():
    T, k, L, E = 3, 2, 8, 5
    idx = np.array([[0, 3], [3, 1], [0, 1]], dtype=np.int32)
    w = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, 0.0]], dtype=np.float32)
    y = np.zeros((T * k, L), dtype=np.float32)
    y[0, 2] = -3.0                 # one-hot: the norm is |value|
    y[1, :2] = (3.0, 4.0)          # a Pythagorean triple: 5
    y[2, 7] = 2.0
    y[3, 0] = 1.5
    y[4, 1], y[4, 5] = 5.0, 12.0   # 13
    y[5, 3] = 7.0                  # weight 0
    s = oracle.reap_saliency(y, w, idx, E)
    assert s[0] == 0.25 * 3.0 + 1.0 * 13.0
    assert s[3] == 0.75 * 5.0 + 0.5 * 2.0
    assert s[1] == 0.5 * 1.5 + 0.0 * 7.0
    assert s[2] == 0.0 and s[4] == 0.0
    assert np.array_equal(oracle.reap_saliency(2 * y, w, idx, E), 2 * s)  # exact power-of-two scaling


def test_saliency_total_and_order_invariance():
    rng = np.random.default_rng(3)
    T, k, L, E = 40, 4, 64, 16
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    y = rng.standard_normal((T * k, L)).astype(np.float32)
    s = oracle.reap_saliency(y, w, idx, E)
    norms = np.linalg.norm(y.astype(np.float64), axis=1)
    assert abs(s.sum() - float((w.reshape(-1).astype(np.float64) * norms).sum())) < 1e-12 * s.sum()
    for e in range(E):
        rows = np.nonzero(idx.reshape(-1) == e)[0]
        assert abs(s[e] - float((w.reshape(-1)[rows].astype(np.float64) * norms[rows]).sum())) <= 1e-12 * max(s[e], 1)
    p = rng.permutation(T)
    yp = y.reshape(T, k, L)[p].reshape(T * k, L)
    sp = oracle.reap_saliency(yp, w[p], idx[p], E)
    assert np.allclose(sp, s, rtol=1e-14, atol=0)


def test_pruned_layer_equals_the_layer_of_the_survivors():
    """A bias of -inf on the pruned experts gives the layer built from the survivors only
    (router rows and records of the kept experts, ids relabelled): same outputs, weights
    renormalised over them."""
    T, d, L, F, E, k = 5, 64, 64, 96, 12, 3
    x = synth.normal_bf16(51, 1, 1.0, (T, d))
    Wr = synth.normal_bf16(51, 2, 0.02, (E, d))
    Wd = synth.normal_bf16(51, 3, 0.02, (L, d))
    Wu = synth.normal_bf16(51, 4, 0.02, (d, L))
    blob = synth.expert_blob(51, L, F, E)
    keep = np.array([1, 2, 4, 7, 8, 11])
    bias = np.full(E, -np.inf, dtype=np.float32)
    bias[keep] = 0.0
    rp = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F, bias=bias)
    assert np.isin(rp["idx"], keep).all()
    assert np.allclose(rp["w"].sum(1), 1.0, atol=1e-6)
    rec = synth.expert_record_bytes(L, F)
    blob_s = np.concatenate([blob[e * rec:(e + 1) * rec] for e in keep])
    rs = oracle.layer_forward(x, np.ascontiguousarray(Wr[keep]), Wd, Wu, blob_s, k, L, F)
    assert np.array_equal(keep[rs["idx"]], rp["idx"])
    assert np.array_equal(rs["w"], rp["w"]) and np.array_equal(rs["out"], rp["out"])


def test_tier_fractions():
    """The REAP tiers keep 242 and 179 of 896 experts (kimi-k3-mlx digest, REAP section):
    27% and 20%, and 27% is also the expected overlap of two random 242-of-896 keep sets,
    the baseline the domain-clustering section measures against (a hypergeometric mean:
    242 x 242 / 896 shared experts).  The keep sets themselves come from GPU saliency in
    the GPU tests (moe_reap_keep_bias, and the prefill32k domain keep sets)."""
    assert round(242 / 896, 2) == 0.27 and round(179 / 896, 2) == 0.20
    assert abs((242 * 242 / 896) / 242 - 0.27) < 0.005


def test_fewer_survivors_than_k_fill_with_zero_weights():
    """Pruned below k (outside the documented precondition): the selection still holds k
    distinct experts, the survivors plus the lowest-index pruned ones (ties at -inf go to
    the lower index), the pruned ones at weight 0 and the survivors' weights their softmax."""
    E, k = 8, 4
    lg = np.full((1, E), -np.inf, dtype=np.float32)
    lg[0, 5], lg[0, 6] = 1.0, 3.0
    idx, w = oracle.select(lg, k)
    assert idx[0].tolist() == [0, 1, 5, 6]
    e = np.exp(np.array([1.0 - 3.0, 0.0]))
    assert w[0, 0] == 0.0 and w[0, 1] == 0.0
    assert np.allclose(w[0, 2:], e / e.sum(), rtol=1e-6, atol=0)
