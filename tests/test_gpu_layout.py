"""Per-expert layout check and decode/batch routing agreement on the GPU.

Every expert of the tiny layer, and experts spread over the whole K3 blob, is applied to a
latent row through moe_expert_ffn (checkpoint and packed layouts) and compared with the
oracle's expert by cosine similarity: a transposed, swapped or mis-stacked matrix drives
it far below the 0.9999 required here (the CPU pin test_expert_cosine_detects_layout_mistakes
shows how far).  The routing of the same tokens one at a time (the GEMV router and the
one-token routing kernel) and as a batch of 40 (the matrix-core router and the batched
routing kernel) must select the same experts.
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import cosine
from gpu_common import dev_packed, dev_weights, from_dev, host_layer, log, to_dev

pytestmark = pytest.mark.gpu

COS_MIN = 0.9999


def _expert_cosines(name, idx, packed):
    T = idx.shape[0]
    h = host_layer(name, T)
    c = h["cfg"]
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    blob = dev_packed(name) if packed else dev_weights(name)["blob"]
    y = from_dev(moe.expert_ffn(to_dev(hl), blob, to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E,
                                packed=packed))
    rec = c.record_bytes
    cos = []
    for t in range(T):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            _, wy = oracle.expert(hl[t], h["blob"][e * rec:(e + 1) * rec], c.L, c.F)
            cos.append(cosine(y[t * idx.shape[1] + j], wy))
    return np.array(cos)


@pytest.mark.parametrize("packed", [False, True])
def test_every_expert_cosine_tiny(packed):
    c = synth.CONFIGS["tiny"]
    # 4 tokens x k = 2: experts 0..7, each row ascending
    idx = np.arange(c.E, dtype=np.int32).reshape(c.E // c.k, c.k)
    cos = _expert_cosines("tiny", idx, packed)
    log(f"  tiny experts: min cosine {cos.min():.7f}")
    assert cos.min() >= COS_MIN


@pytest.mark.parametrize("packed", [False, True])
def test_k3_experts_cosine_spread_over_the_blob(packed):
    c = synth.CONFIGS["decode1"]
    # 2 tokens x k = 16: 32 experts spread over all 896 (every 29th from 0, and the last)
    ids = np.concatenate([np.arange(0, c.E, 29)[:31], [c.E - 1]])
    assert ids.size == 32 and np.all(np.diff(ids) > 0)
    idx = ids.reshape(2, 16).astype(np.int32)
    cos = _expert_cosines("decode1", idx, packed)
    log(f"  K3 experts {ids[0]}..{ids[-1]}: min cosine {cos.min():.7f}")
    assert cos.min() >= COS_MIN


@pytest.mark.parametrize("name", ["tiny", "decode64"])
def test_routing_one_token_and_batch_agree(name):
    """Routing is exact, so the decode path (T = 1) and the batched path (T = 40) select the
    same experts for the same tokens, and both equal the oracle's selection."""
    h = host_layer(name, 40)
    c = h["cfg"]
    dw = dev_weights(name)
    x = h["x"][:40]

    def run(xs):
        idx = torch.empty((xs.shape[0], c.k), dtype=torch.int32, device="cuda")
        moe.layer_forward(to_dev(xs), dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k,
                          d_ffn=c.F, routing={"topk_idx": idx})
        return from_dev(idx)

    batch = run(x)
    one = np.concatenate([run(x[t:t + 1]) for t in range(8)])
    assert np.array_equal(one, batch[:8])
    want, _ = oracle.select(oracle.router_logits(x, h["router_w"], None), c.k)
    assert np.array_equal(batch, want)
