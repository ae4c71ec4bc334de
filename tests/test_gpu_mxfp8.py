"""The MXFP8-activation mode (moe_config.act_format = MOE_ACT_FMT_MXFP8) against the
oracle's MXFP8 mode: the latent rows h and the GLU rows a are quantised to E4M3 with
an e8m0 scale per 32 (OCP MX convention) on both sides, the same codes from the same
bf16 values; sums differ only in order, so the bf16-mode tolerance applies."""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import bf16_bits_to_f64, rel_l2
from gpu_common import ORACLE_THREADS, dev_packed, dev_weights, from_dev, host_layer, log, oracle_routing, to_dev

pytestmark = pytest.mark.gpu

TOL_OUT = 2e-3


def _run(name, T=None, tokens=None, packed=True):
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    blob = dev_packed(name) if packed else dw["blob"]
    Tn = h["x"].shape[0]
    idx = torch.empty((Tn, c.k), dtype=torch.int32, device="cuda")
    out = moe.layer_forward(to_dev(h["x"]), dw["router_w"], dw["latent_down"], dw["latent_up"], blob, c.k,
                            d_ffn=c.F, bias=None if h["bias"] is None else to_dev(h["bias"]),
                            routing={"topk_idx": idx}, packed=packed, act_format=moe.ACT_FMT_MXFP8)
    out = from_dev(out)
    tokens = list(range(Tn)) if tokens is None else tokens
    ref = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                               bias=h["bias"], tokens=tokens, act_format=oracle.ACT_MXFP8, threads=ORACLE_THREADS)
    assert np.array_equal(from_dev(idx)[tokens], ref["idx"])
    if T is None and c.d == 7168:  # the routing does not depend on the activation format
        assert np.array_equal(from_dev(idx), oracle_routing(name)[1])
    err = rel_l2(bf16_bits_to_f64(out[tokens]), bf16_bits_to_f64(ref["out"]))
    # the bf16-mode oracle, for scale: the mode really quantises
    ref_b = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L,
                                 c.F, bias=h["bias"], tokens=tokens, threads=ORACLE_THREADS)
    dev_b = rel_l2(bf16_bits_to_f64(out[tokens]), bf16_bits_to_f64(ref_b["out"]))
    log(f"  {name} T={Tn} MXFP8 rel-L2 = {err:.3g} (against the bf16 mode: {dev_b:.3g})")
    assert err <= TOL_OUT
    assert dev_b > 5 * TOL_OUT


@pytest.mark.parametrize("packed", [False, True])
def test_layer_mxfp8_tiny(packed):
    _run("tiny", packed=packed)


@pytest.mark.parametrize("T", [40, 600, 1100])
def test_layer_mxfp8_tiny_every_dispatch_path(T):
    """Streaming kernels (40 tokens) and grouped GEMMs (600, 1100) on the tiny layer."""
    _run("tiny", T=T, tokens=[0, 1, T // 2, T - 1])


def test_layer_mxfp8_decode1():
    _run("decode1")


def test_layer_mxfp8_decode64_every_token():
    _run("decode64")


def test_layer_mxfp8_prefill4k_sampled():
    _run("prefill4k", tokens=[0, 2047, 4095])


def test_layer_mxfp8_prefill32k_sampled():
    """The prompt cap in the MXFP8 mode: every token's routing, outputs on a sample."""
    rng = np.random.default_rng(0x8F8)
    _run("prefill32k", tokens=sorted({0, 32767, *rng.choice(32768, 14, replace=False).tolist()}))


def test_expert_ffn_mxfp8_rows():
    """The expert stage alone on given h and routing, row by row against the oracle."""
    h = host_layer("decode64", 8)
    c = h["cfg"]
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    idx, _ = oracle.select(oracle.router_logits(h["x"], h["router_w"], h["bias"]), c.k)
    y, a = moe.expert_ffn(to_dev(hl), dev_packed("decode64"), to_dev(idx), d_model=c.d, d_ffn=c.F,
                          num_experts=c.E, want_a=True, packed=True, act_format=moe.ACT_FMT_MXFP8)
    y = from_dev(y)
    rec = c.record_bytes
    errs = []
    for t in (0, 7):
        for j in (0, c.k - 1):
            e = int(idx[t, j])
            _, yr = oracle.expert(hl[t], h["blob"][e * rec:(e + 1) * rec], c.L, c.F, act_format=oracle.ACT_MXFP8)
            errs.append(rel_l2(y[t * c.k + j].astype(np.float64), yr.astype(np.float64)))
    log(f"  expert rows MXFP8 rel-L2 max {max(errs):.3g}")
    assert max(errs) <= TOL_OUT
