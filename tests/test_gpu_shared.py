"""Shared experts (moe_layer_forward_shared) against the oracle: SiLU-GLU experts on the
full-width token, weight 1, added to the latent-up product before the output rounding."""
import functools

import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import bf16_bits_to_f64, rel_l2
from gpu_common import dev_packed, dev_weights, from_dev, host_layer, log, to_dev

pytestmark = pytest.mark.gpu

TOL_OUT = 2e-3
S = 2


@functools.lru_cache(maxsize=None)
def _shared(d, F_s):
    return synth.expert_blob(0x5A4ED + d, d, F_s, S)


def _run(name, T=None, tokens=None, packed=True, act_format=0):
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    F_s = c.F
    sh = _shared(c.d, F_s)
    dsh = to_dev(sh)
    if packed:
        dsh = moe.pack_experts(dsh, S, c.d, F_s)
    blob = dev_packed(name) if packed else dw["blob"]
    Tn = h["x"].shape[0]
    out = moe.layer_forward(to_dev(h["x"]), dw["router_w"], dw["latent_down"], dw["latent_up"], blob, c.k,
                            d_ffn=c.F, bias=None if h["bias"] is None else to_dev(h["bias"]), packed=packed,
                            act_format=act_format, shared_blob=dsh, num_shared=S, d_ffn_shared=F_s)
    out = from_dev(out)
    tokens = list(range(Tn)) if tokens is None else tokens
    ref = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                               bias=h["bias"], tokens=tokens, act_format=act_format, shared_blob=sh, num_shared=S,
                               d_ffn_shared=F_s)
    err = rel_l2(bf16_bits_to_f64(out[tokens]), bf16_bits_to_f64(ref["out"]))
    plain = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                                 bias=h["bias"], tokens=tokens, act_format=act_format)
    moved = rel_l2(bf16_bits_to_f64(ref["out"]), bf16_bits_to_f64(plain["out"]))
    log(f"  {name} T={Tn} shared x{S}: rel-L2 {err:.3g} (the shared experts move the output by {moved:.3g})")
    assert err <= TOL_OUT
    assert moved > 10 * TOL_OUT


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("T", [None, 40, 600])
def test_layer_shared_tiny(packed, T):
    _run("tiny", T=T, tokens=None if T is None else [0, 1, T // 2, T - 1], packed=packed)


def test_layer_shared_tiny_mxfp8():
    _run("tiny", T=600, tokens=[0, 599], act_format=moe.ACT_FMT_MXFP8)


def test_layer_shared_decode1():
    _run("decode1")


def test_layer_shared_prefill4k_sampled():
    _run("prefill4k", tokens=[0, 4095])


def test_shared_requires_the_blob():
    h = host_layer("tiny")
    c = h["cfg"]
    dw = dev_weights("tiny")
    cfg = moe.make_config(16, c.d, c.L, c.F, c.E, num_shared=2, d_ffn_shared=c.F)
    ws = moe.alloc_workspace(cfg, c.k, torch.device("cuda"))
    out = torch.empty((16, c.d), dtype=torch.int16, device="cuda")
    st = moe.lib().moe_layer_forward(to_dev(h["x"]).data_ptr(), dw["router_w"].data_ptr(),
                                     dw["latent_down"].data_ptr(), dw["latent_up"].data_ptr(), dw["blob"].data_ptr(),
                                     c.k, __import__("ctypes").byref(cfg), None, out.data_ptr(), None, ws.data_ptr(),
                                     ws.numel(), None)
    assert st == -1


def test_layer_shared_prefill32k_sampled():
    _run("prefill32k", tokens=[0, 16383, 32767])


@pytest.mark.parametrize("name,T", [("decode1", None), ("tiny", 600)])
def test_layer_shared_graph_replays_match_eager(name, T):
    """The shared experts run on the library's second stream, forked from the caller's
    stream and joined before the latent-up projection.  Captured into a graph (whose
    capture stream differs from the eager call's), every replay, with other work on the
    device between replays, gives the eager call's bits."""
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    dsh = moe.pack_experts(to_dev(_shared(c.d, c.F)), S, c.d, c.F)
    blob = dev_packed(name)
    Tn = h["x"].shape[0]
    x = to_dev(h["x"])
    bias = None if h["bias"] is None else to_dev(h["bias"])
    cfg = moe.make_config(Tn, c.d, c.L, c.F, c.E, num_shared=S, d_ffn_shared=c.F, packed=True)
    ws = moe.alloc_workspace(cfg, c.k, torch.device("cuda"))
    out = torch.empty((Tn, c.d), dtype=torch.int16, device="cuda")

    def call():
        moe.layer_forward(x, dw["router_w"], dw["latent_down"], dw["latent_up"], blob, c.k, d_ffn=c.F, bias=bias,
                          packed=True, shared_blob=dsh, num_shared=S, d_ffn_shared=c.F, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        call()  # eager work between replays, on the same buffers
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    log(f"  {name} T={Tn}: 3 graph replays bit-identical to the eager call")
