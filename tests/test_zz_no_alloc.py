"""moe_layer_forward_noalloc, the entry point for callers that cannot allocate: through the
C ABI, on two calls in a row (the second with a smaller batch, so it runs on the scratch
the first left behind), its outputs and routing equal moe_layer_forward's bit for bit
(same kernels, same inputs), and a batch past the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import synth
from gpu_common import dev_weights, from_dev, host_layer, log, to_dev

pytestmark = pytest.mark.gpu


def _routing(T, c):
    return dict(topk_idx=torch.empty((T, c.k), dtype=torch.int32, device="cuda"),
                topk_w=torch.empty((T, c.k), dtype=torch.float32, device="cuda"),
                logits=torch.empty((T, c.E), dtype=torch.float32, device="cuda"),
                expert_counts=torch.empty(c.E, dtype=torch.int32, device="cuda"),
                expert_offsets=torch.empty(c.E + 1, dtype=torch.int32, device="cuda"),
                perm=torch.empty(T * c.k, dtype=torch.int32, device="cuda"))


def _both(name, x, bias, packed=False):
    c = synth.CONFIGS[name]
    dw = dev_weights(name)
    T = x.shape[0]
    res = []
    for noalloc in (False, True):
        r = _routing(T, c)
        out = torch.empty((T, c.d), dtype=torch.int16, device="cuda")
        args = (to_dev(x), dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k)
        kw = dict(d_ffn=c.F, bias=None if bias is None else to_dev(bias), out=out, routing=r)
        if noalloc:
            moe.layer_forward_noalloc(*args, **kw)
        else:
            moe.layer_forward(*args, **kw)
        torch.cuda.synchronize()
        res.append([from_dev(out)] + [from_dev(v) for v in r.values()])
    return res


def _same(a, b):
    return all(np.array_equal(u.view(np.uint8), v.view(np.uint8)) for u, v in zip(a, b))


@pytest.mark.parametrize("name,T1,T2", [("tiny", 16, 3), ("decode64", 64, 5)])
def test_noalloc_equals_layer_forward_two_calls(name, T1, T2):
    """A batch, then a smaller one on the same scratch: both equal moe_layer_forward."""
    h = host_layer(name)
    c = h["cfg"]
    for T in (T1, T2):
        x = np.ascontiguousarray(h["x"][:T]) if T <= h["x"].shape[0] else synth.make_tokens(c, T=T)
        ref, got = _both(name, x, h["bias"])
        log(f"  {name} T={T}: noalloc equals layer_forward: {_same(ref, got)}")
        assert _same(ref, got), (name, T)


def test_noalloc_prefill_shapes_with_bias_after_a_larger_batch():
    """Tokens of the 4096-token prefill workload (router bias, certified routing of several
    tokens per block): 128 tokens, then 7 on the scratch the 128 left."""
    c = synth.CONFIGS["prefill4k"]
    h = host_layer("prefill4k", 128)
    for T in (128, 7):
        x = np.ascontiguousarray(h["x"][:T])
        ref, got = _both("prefill4k", x, h["bias"])
        assert _same(ref, got), T
    assert moe.workspace_size(moe.make_config(128, c.d, c.L, c.F, c.E), c.k) <= moe.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_a_batch_past_the_scratch():
    """4096 K3 tokens need more than the scratch: MOE_ERR_WORKSPACE, nothing written."""
    c = synth.CONFIGS["prefill4k"]
    dw = dev_weights("prefill4k")
    assert moe.workspace_size(moe.make_config(4096, c.d, c.L, c.F, c.E), c.k) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((4096, c.d), dtype=torch.int16, device="cuda")
    out = torch.full((4096, c.d), 0x1234, dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.layer_forward_noalloc(x, dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k, d_ffn=c.F,
                                  out=out)
    assert ei.value.status == -3
    torch.cuda.synchronize()
    assert (out == 0x1234).all()
