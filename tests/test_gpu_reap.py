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
