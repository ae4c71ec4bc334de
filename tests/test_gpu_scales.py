"""Expert records with e8m0 scales at the edges of the format, through the matrix-core
expert kernels (the MXFP4 scale bytes go to the block-scaled MFMA as they are stored).

Scale byte s means 2^(s-127) for s = 0..254 and NaN for 255 (kimi-k3-in-c post, MXFP4
section: one 8-bit exponent per 32 weights; OCP Microscaling v1.0 for the encoding).  The
oracle multiplies by the weights' exact values.  Each expert below pairs a scale range
with latent rows whose magnitude keeps the fp32 sums in range, so every finite value can
be compared: both ends of the range (0, 1-20, 235-254, where the largest weights of
scales 253-254 lie past the fp32 range), and NaN blocks in gate, up and down.  Results
are compared element by element: NaN in the same positions, infinities in the same
positions with the same sign, finite values to the usual tolerance.
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import bf16_bits_to_f64, f64_to_bf16_bits, rel_l2
from gpu_common import from_dev, log, to_dev

pytestmark = pytest.mark.gpu

L = F = 128
E, K = 8, 2

# per expert: (gate/up scale range, down scale range, NaN blocks as (matrix, scale index))
EXPERTS = [
    ((0, 0), (120, 130), []),          # 0: gate/up at 2^-127 (weights down to 2^-128)
    ((1, 20), (1, 20), []),            # 1: the low end everywhere
    ((235, 254), (120, 130), []),      # 2: the high end on gate/up
    ((60, 80), (235, 254), []),        # 3: the high end on down
    ((120, 130), (120, 130), [(0, 9)]),   # 4: one NaN block in gate
    ((120, 130), (120, 130), [(2, 17)]),  # 5: one NaN block in down
    ((120, 130), (120, 130), [(1, 30)]),  # 6: one NaN block in up
    ((120, 130), (120, 130), []),      # 7: the generator's range
]
# per token: (exponent of its latent row's magnitude, its two experts)
TOKENS = [(100, [0, 1]), (-100, [2, 7]), (0, [3, 4]), (0, [5, 6]), (0, [4, 7]), (100, [0, 1])]


def edge_blob(seed=0xE8):
    nc, ns = F * L // 2, F * L // 32
    mat = nc + ns
    rec = synth.expert_record_bytes(L, F)
    blob = synth.expert_blob(seed, L, F, E)
    rng = np.random.default_rng(seed)
    for e, (gu, dn, nans) in enumerate(EXPERTS):
        r = blob[e * rec:(e + 1) * rec]
        for m, (lo, hi) in enumerate((gu, gu, dn)):
            r[m * mat + nc:(m + 1) * mat] = rng.integers(lo, hi + 1, ns)
        for m, b in nans:
            r[m * mat + nc + b] = 255
    return blob


def edge_rows(reps=1, seed=0xE9):
    rng = np.random.default_rng(seed)
    hs, idx = [], []
    for _ in range(reps):
        for ex, ids in TOKENS:
            hs.append(f64_to_bf16_bits(rng.standard_normal(L) * 2.0 ** ex))
            idx.append(ids)
    return np.stack(hs), np.array(idx, dtype=np.int32)


def _classes(v):
    v = np.asarray(v, np.float64)
    return np.isnan(v), np.isposinf(v), np.isneginf(v)


def compare_rows(y, a, yo, ao, what):
    """y fp32, a bf16 bits of one routed row against the oracle's; returns the y error."""
    fy, fyo = y.astype(np.float64), yo.astype(np.float64)
    fa, fao = bf16_bits_to_f64(a), bf16_bits_to_f64(ao)
    for name, g, o in (("y", fy, fyo), ("a", fa, fao)):
        for cls, gm, om in zip(("NaN", "+inf", "-inf"), _classes(g), _classes(o)):
            assert np.array_equal(gm, om), f"{what}: {name} {cls} at {np.nonzero(gm != om)[0][:8]}"
    fin = np.isfinite(fao)
    ulps = np.abs(a[fin].astype(np.int64) - ao[fin].astype(np.int64))
    assert np.mean(ulps <= 1) >= 0.98, f"{what}: a within one ulp {np.mean(ulps <= 1):.3f}"
    fin = np.isfinite(fyo)
    err = rel_l2(fy[fin], fyo[fin]) if fin.any() and np.any(fyo[fin] != 0) else float(np.max(np.abs(fy[fin]), initial=0))
    assert err < 1e-3, f"{what}: y rel-L2 {err:.3g}"
    return err


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("reps", [1, 11])
def test_expert_ffn_edge_scales(packed, reps):
    """12 routed rows take the streaming kernels, 132 (at least 8 per expert on average)
    the grouped GEMMs."""
    blob = edge_blob()
    h, idx = edge_rows(reps)
    db = to_dev(blob)
    if packed:
        db = moe.pack_experts(db, E, L, F)
    y, a = moe.expert_ffn(to_dev(h), db, to_dev(idx), d_model=256, d_ffn=F, num_experts=E, want_a=True,
                          packed=packed)
    y, a = from_dev(y), from_dev(a)
    rec = synth.expert_record_bytes(L, F)
    errs = {}
    for t in range(h.shape[0]):
        for j in range(K):
            e = int(idx[t, j])
            ao, yo = oracle.expert(h[t], blob[e * rec:(e + 1) * rec], L, F)
            errs[e] = max(errs.get(e, 0.0), compare_rows(y[t * K + j], a[t * K + j], yo, ao,
                                                         f"token {t} expert {e}"))
    log(f"  packed={packed} rows={h.shape[0] * K}: y rel-L2 by expert " +
        ", ".join(f"{e}:{v:.2g}" for e, v in sorted(errs.items())))
    # the NaN blocks reach the outputs as the format defines
    y3 = y.reshape(-1, K, L)
    assert np.isnan(y3[2, 1]).all()          # token 2, expert 4 (NaN in gate): every y NaN
    row = 17 // (F // 32)
    assert np.isnan(y3[3, 0, row]) and np.isfinite(np.delete(y3[3, 0], row)).all()  # expert 5: one row


@pytest.mark.parametrize("T", [16, 600])
def test_layer_tiny_edge_scales(T):
    """The tiny layer (routing, latent projections, combine) over the edge-scale experts:
    routing bit-exact; tokens routed to an expert whose output holds NaN come out NaN on
    both sides, the others within the layer tolerance."""
    c = synth.CONFIGS["tiny"]
    d = synth.make_dense(c)
    blob = edge_blob()
    x = synth.make_tokens(c, T=T)
    idx = torch.empty((T, c.k), dtype=torch.int32, device="cuda")
    out = moe.layer_forward(to_dev(x), to_dev(d["router_w"]), to_dev(d["latent_down"]), to_dev(d["latent_up"]),
                            to_dev(blob), c.k, d_ffn=c.F, routing={"topk_idx": idx})
    out = from_dev(out)
    ref = oracle.layer_forward(x, d["router_w"], d["latent_down"], d["latent_up"], blob, c.k, c.L, c.F)
    assert np.array_equal(from_dev(idx), ref["idx"])
    g, o = bf16_bits_to_f64(out), bf16_bits_to_f64(ref["out"])
    for cls, gm, om in zip(("NaN", "+inf", "-inf"), _classes(g), _classes(o)):
        assert np.array_equal(gm, om), f"{cls} rows differ: {np.nonzero((gm != om).any(1))[0][:8]}"
    fin = np.isfinite(o).all(1)
    log(f"  T={T}: {int((~fin).sum())} tokens with non-finite outputs, "
        f"rel-L2 over the others {rel_l2(g[fin], o[fin]):.3g}")
    assert (~fin).any() and fin.any()
    assert rel_l2(g[fin], o[fin]) <= 2e-3
