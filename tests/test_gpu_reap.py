"""REAP on the GPU: the saliency accumulation against the oracle's, and a pruned layer
(bias -inf on the removed experts) routed exactly with renormalised weights."""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import bf16_bits_to_f64, rel_l2
from gpu_common import dev_packed, dev_weights, from_dev, host_layer, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("tiny", 600), ("decode64", None)])
def test_reap_saliency_matches_oracle(name, T):
    h = host_layer(name, T)
    c = h["cfg"]
    Tn = h["x"].shape[0]
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    idx, w = oracle.select(oracle.router_logits(h["x"], h["router_w"], h["bias"]), c.k)
    blob = dev_weights(name)["blob"]
    y = moe.expert_ffn(to_dev(hl), blob, to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E)
    counts, offsets, perm = moe.permute(to_dev(idx), c.E)
    s = moe.reap_saliency(y, to_dev(w), perm, offsets, c.E)
    s = moe.reap_saliency(y, to_dev(w), perm, offsets, c.E, saliency=s)  # accumulates
    want = oracle.reap_saliency(from_dev(y), w, idx, c.E)
    got = from_dev(s)
    log(f"  {name} T={Tn}: max rel dev {np.max(np.abs(got - 2 * want) / np.maximum(2 * want, 1e-30)):.3g}")
    assert np.allclose(got, 2 * want, rtol=1e-12, atol=0)
    assert (got[np.bincount(idx.reshape(-1), minlength=c.E) == 0] == 0).all()


@pytest.mark.parametrize("name,T,n_keep", [("decode1", None, 242), ("decode64", None, 179), ("prefill4k", 256, 242)])
def test_pruned_layer_routes_exactly(name, T, n_keep):
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    rng = np.random.default_rng(c.E + n_keep)
    keep = np.sort(rng.choice(c.E, n_keep, replace=False))
    bias = np.full(c.E, -np.inf, dtype=np.float32)
    if h["bias"] is not None and h["bias"].ndim == 1:
        bias[keep] = h["bias"][keep]
    else:
        bias[keep] = 0.0
    Tn = h["x"].shape[0]
    idx = torch.empty((Tn, c.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((Tn, c.k), dtype=torch.float32, device="cuda")
    out = moe.layer_forward(to_dev(h["x"]), dw["router_w"], dw["latent_down"], dw["latent_up"], dev_packed(name),
                            c.k, d_ffn=c.F, bias=to_dev(bias), routing={"topk_idx": idx, "topk_w": wts},
                            packed=True)
    gi, gw = from_dev(idx), from_dev(wts)
    assert np.isin(gi, keep).all()
    assert np.allclose(gw.sum(1), 1.0, atol=1e-5)
    lg = oracle.router_logits(h["x"], h["router_w"], bias)
    want_idx, want_w = oracle.select(lg, c.k)
    assert np.array_equal(gi, want_idx)
    assert np.allclose(gw, want_w, rtol=1e-4, atol=1e-6)
    tokens = [0] if Tn == 1 else [0, Tn - 1]
    ref = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                               bias=bias, tokens=tokens)
    err = rel_l2(bf16_bits_to_f64(from_dev(out)[tokens]), bf16_bits_to_f64(ref["out"]))
    log(f"  {name} keep {n_keep}: rel-L2 {err:.3g}")
    assert err <= 2e-3


@pytest.mark.parametrize("name,T,n_keep", [("tiny", 5, 1), ("decode1", None, 10)])
def test_pruned_below_k_fills_with_zero_weight_experts(name, T, n_keep):
    """Fewer survivors than k: every survivor is selected, the remaining slots take the
    lowest-numbered pruned experts (ties at -inf go to the lower index) at weight 0, as
    the oracle selects, and the layer output is the survivors' mixture."""
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    rng = np.random.default_rng(c.E * 7 + n_keep)
    keep = np.sort(rng.choice(c.E, n_keep, replace=False))
    bias = np.full(c.E, -np.inf, dtype=np.float32)
    bias[keep] = 0.0
    Tn = h["x"].shape[0]
    idx = torch.empty((Tn, c.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((Tn, c.k), dtype=torch.float32, device="cuda")
    out = moe.layer_forward(to_dev(h["x"]), dw["router_w"], dw["latent_down"], dw["latent_up"], dev_packed(name),
                            c.k, d_ffn=c.F, bias=to_dev(bias), routing={"topk_idx": idx, "topk_w": wts},
                            packed=True)
    gi, gw = from_dev(idx), from_dev(wts)
    lg = oracle.router_logits(h["x"], h["router_w"], bias)
    want_idx, want_w = oracle.select(lg, c.k)
    assert np.array_equal(gi, want_idx)
    pruned = ~np.isin(gi, keep)
    assert pruned.sum() == Tn * (c.k - n_keep) and (gw[pruned] == 0).all()
    assert np.allclose(gw, want_w, rtol=1e-4, atol=1e-6)
    tokens = [0] if Tn == 1 else [0, Tn - 1]
    ref = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                               bias=bias, tokens=tokens)
    err = rel_l2(bf16_bits_to_f64(from_dev(out)[tokens]), bf16_bits_to_f64(ref["out"]))
    log(f"  {name} keep {n_keep} < k: rel-L2 {err:.3g}")
    assert err <= 2e-3


def _routing_bufs(Tn, k, E):
    z = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device="cuda")
    return {"topk_idx": z(Tn, k), "topk_w": z(Tn, k, dt=torch.float32), "expert_counts": z(E),
            "expert_offsets": z(E + 1), "perm": z(Tn * k),
            "saliency": torch.zeros(E, dtype=torch.float64, device="cuda")}


@pytest.mark.parametrize("name,T,packed,fmt", [("decode1", None, True, 0), ("decode64", None, True, 0),
                                               ("decode64", None, False, 0), ("tiny", 600, True, 0),
                                               ("tiny", 600, True, 1), ("prefill4k", None, True, 0)])
def test_layer_saliency_fused_matches_the_oracle(name, T, packed, fmt):
    """The layer's REAP sums (partials written by the down kernel that runs: the fused
    down+combine at decode1, the streaming down at decode64, the grouped GEMM at tiny 600
    and prefill4k) against the oracle's moe_ref_reap_saliency on the same y, taken from
    moe_expert_ffn with the layer's routing, and against the separate saliency kernel.
    Two calls accumulate twice the sums."""
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    Tn = h["x"].shape[0]
    x = to_dev(h["x"])
    r = _routing_bufs(Tn, c.k, c.E)
    blob = dev_packed(name) if packed else dw["blob"]
    bias = None if h["bias"] is None else to_dev(h["bias"])
    for _ in range(2):
        moe.layer_forward(x, dw["router_w"], dw["latent_down"], dw["latent_up"], blob, c.k, d_ffn=c.F, bias=bias,
                          routing=r, packed=packed, act_format=fmt)
    got = from_dev(r["saliency"]) / 2
    hl = moe.linear_bf16(x, dw["latent_down"])
    y = moe.expert_ffn(hl, blob, r["topk_idx"], d_model=c.d, d_ffn=c.F, num_experts=c.E, packed=packed,
                       act_format=fmt)
    sep = from_dev(moe.reap_saliency(y, r["topk_w"], r["perm"], r["expert_offsets"], c.E))
    want = oracle.reap_saliency(from_dev(y), from_dev(r["topk_w"]), from_dev(r["topk_idx"]), c.E)
    dev_o = np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-300))
    dev_s = np.max(np.abs(got - sep) / np.maximum(np.abs(sep), 1e-300))
    log(f"  {name} T={Tn} packed={packed} fmt={fmt}: {int((want > 0).sum())} experts scored, "
        f"max rel dev {dev_o:.3g} (oracle), {dev_s:.3g} (separate kernel)")
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    assert np.allclose(got, sep, rtol=1e-12, atol=0)
    assert (got[from_dev(r["expert_counts"]) == 0] == 0).all()


def test_keep_bias_ranks_like_a_stable_sort():
    """moe_reap_keep_bias against numpy: higher saliency first, ties to the lower index,
    NaN after every number; n_keep from 0 to E."""
    rng = np.random.default_rng(7)
    E = 896
    s = rng.integers(0, 50, E).astype(np.float64)  # many ties
    s[rng.choice(E, 20, replace=False)] = np.nan
    s[rng.choice(E, 5, replace=False)] = -np.inf
    s[3], s[4] = 0.0, -0.0
    order = sorted(range(E), key=lambda e: (np.isnan(s[e]), -s[e] if not np.isnan(s[e]) else 0.0, e))
    ds = to_dev(s)
    for n_keep in (0, 1, 179, 242, 895, 896):
        b = from_dev(moe.reap_prune_bias(ds, n_keep))
        want = np.full(E, -np.inf, dtype=np.float32)
        want[order[:n_keep]] = 0.0
        assert np.array_equal(b, want), n_keep


def test_prefill32k_domain_keep_sets():
    """Keep sets of 242 experts from GPU saliency on each of prefill32k's four token
    domains (each favours its own 224-expert cluster), and on two halves of each domain
    (kimi-k3-mlx digest, domain-clustering section: keep sets of different corpora are
    compared against the 27% overlap of two random 242-of-896 sets).  Halves of one domain
    agree far above that baseline, different domains fall below it, and each keep set holds
    its domain's cluster."""
    h = host_layer("prefill32k")
    c = h["cfg"]
    dw = dev_weights("prefill32k")
    blob = dev_packed("prefill32k")
    dom_key = np.argmax(h["bias"], axis=1)  # the first expert of the token's cluster
    doms = np.unique(dom_key)
    assert len(doms) == 4
    base = 242 / 896

    def keep_set(rows):
        x = to_dev(np.ascontiguousarray(h["x"][rows]))
        bias = to_dev(np.ascontiguousarray(h["bias"][rows]))
        r = _routing_bufs(len(rows), c.k, c.E)
        moe.layer_forward(x, dw["router_w"], dw["latent_down"], dw["latent_up"], blob, c.k, d_ffn=c.F, bias=bias,
                          routing=r, packed=True)
        b = from_dev(moe.reap_prune_bias(r["saliency"], 242))
        sal = from_dev(r["saliency"])
        order = sorted(range(c.E), key=lambda e: (-sal[e], e))
        assert set(np.nonzero(b == 0)[0]) == set(order[:242])
        return set(np.nonzero(b == 0)[0].tolist())

    full, halves = {}, {}
    for d in doms:
        rows = np.nonzero(dom_key == d)[0]
        full[d] = keep_set(rows)
        halves[d] = (keep_set(rows[0::2]), keep_set(rows[1::2]))
        cluster = set(np.nonzero(h["bias"][rows[0]] == 2.0)[0].tolist())
        held = len(full[d] & cluster) / len(cluster)
        within = len(halves[d][0] & halves[d][1]) / 242
        log(f"  domain {d}: {len(rows)} tokens, keep set holds {held:.1%} of its cluster, halves overlap {within:.1%}")
        assert held > 0.9
        assert within > 2 * base
    for i, a in enumerate(doms):
        for b_ in doms[i + 1:]:
            ov = len(full[a] & full[b_]) / 242
            log(f"  domains {a} and {b_}: overlap {ov:.1%} (random baseline {base:.1%})")
            assert ov < base
