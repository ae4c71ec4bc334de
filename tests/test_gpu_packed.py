"""The packed expert layout (moe_pack_experts): the packed bytes follow the layout the
header defines, and the layer and expert stage give bit-identical results on the packed
and on the checkpoint layout (the matrix-core operands are the same bytes)."""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import bf16_bits_to_f64, rel_l2
from gpu_common import ORACLE_THREADS, dev_packed, dev_weights, from_dev, host_layer, log, oracle_routing, to_dev

pytestmark = pytest.mark.gpu


def pack_reference(blob: np.ndarray, E: int, L: int, F: int) -> np.ndarray:
    """The packed layout written out from its definition in include/moe_layer.h."""
    out = []
    rec = F * L // 2 * 3 + F * L // 32 * 3
    for e in range(E):
        r = blob[e * rec:(e + 1) * rec]
        off = 0
        for R, K in ((F, L), (F, L), (L, F)):
            codes = r[off:off + R * K // 2].reshape(R, K // 2)
            scales = r[off + R * K // 2:off + R * K // 2 + R * K // 32].reshape(R, K // 32)
            off += R * K // 2 + R * K // 32
            nks = K // 128
            nsc = (nks + 3) // 4
            for grp in range(R // 16):
                rows = slice(16 * grp, 16 * grp + 16)
                # code tile s: lane l = n + 16 b holds row n, bytes 64 s + 16 b .. +15
                c = codes[rows].reshape(16, nks, 4, 16)          # [n][s][b][byte]
                out.append(c.transpose(1, 2, 0, 3).reshape(-1))  # [s][b][n][byte]
                # scale tile t: byte 4 l + j = scale of row n, block 4 (4 t + j) + b
                sc = np.full((16, 4 * nsc, 4), 127, dtype=np.uint8)
                sc[:, :nks, :] = scales[rows].reshape(16, nks, 4)  # [n][s][b]
                sc = sc.reshape(16, nsc, 4, 4)                       # [n][t][j][b]
                out.append(sc.transpose(1, 3, 0, 2).reshape(-1))     # [t][b][n][j]
    return np.concatenate(out)


@pytest.mark.parametrize("E,L,F", [(3, 384, 256), (2, 128, 128), (2, 512, 640)])
def test_pack_matches_layout_definition(E, L, F):
    blob = synth.expert_blob(0xFACE + L, L, F, E)
    got = from_dev(moe.pack_experts(to_dev(blob), E, L, F))
    want = pack_reference(blob, E, L, F)
    assert got.size == E * moe.packed_expert_bytes(L, F) == want.size
    assert np.array_equal(got, want)


def test_pack_k3_record_sizes_and_bytes():
    """The K3 records keep their size and the first and last experts pack as defined."""
    c = synth.CONFIGS["decode1"]
    assert moe.packed_expert_bytes(c.L, c.F) == moe.expert_bytes(c.L, c.F) == 17547264
    packed = dev_packed("decode1")
    blob = host_layer("decode1")["blob"]
    rec = c.record_bytes
    for e in (0, c.E - 1):
        want = pack_reference(blob[e * rec:(e + 1) * rec], 1, c.L, c.F)
        assert np.array_equal(from_dev(packed[e * rec:(e + 1) * rec]), want)


def _both_layouts(name, x, bias=None, T=None):
    c = synth.CONFIGS[name]
    dw = dev_weights(name)
    outs = []
    for packed in (False, True):
        blob = dev_packed(name) if packed else dw["blob"]
        idx = torch.empty((x.shape[0], c.k), dtype=torch.int32, device="cuda")
        out = moe.layer_forward(to_dev(x), dw["router_w"], dw["latent_down"], dw["latent_up"], blob, c.k,
                                d_ffn=c.F, bias=None if bias is None else to_dev(bias), routing={"topk_idx": idx},
                                packed=packed)
        outs.append((from_dev(out), from_dev(idx)))
    return outs


@pytest.mark.parametrize("T", [1, 5, 40, 600, 1100])
def test_layer_packed_bit_identical_tiny(T):
    c = synth.CONFIGS["tiny"]
    x = synth.make_tokens(c, T=T)
    (a, ia), (b, ib) = _both_layouts("tiny", x)
    assert np.array_equal(ia, ib) and np.array_equal(a, b)


@pytest.mark.parametrize("name,T", [("decode1", None), ("decode64", None), ("prefill4k", 64), ("prefill4k", None),
                                    ("prefill32k", None)])
def test_layer_packed_k3(name, T):
    """Both layouts bit-identical on the K3 workloads, up to the prompt cap (the packed
    layout is the benchmark's default); the packed result against the oracle: every
    token's routing, outputs on the first, middle and last tokens."""
    h = host_layer(name, T)
    c = h["cfg"]
    (a, ia), (b, ib) = _both_layouts(name, h["x"], h["bias"])
    assert np.array_equal(ia, ib) and np.array_equal(a, b)
    n = h["x"].shape[0]
    tokens = sorted({0, n // 2, n - 1})
    if T is None:
        assert np.array_equal(ib, oracle_routing(name)[1])
    ref = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                               bias=h["bias"], tokens=tokens, threads=ORACLE_THREADS)
    err = rel_l2(bf16_bits_to_f64(b[tokens]), bf16_bits_to_f64(ref["out"]))
    log(f"  {name} packed rel-L2 = {err:.3g}")
    assert np.array_equal(ib[tokens], ref["idx"]) and err <= 2e-3


def test_expert_ffn_packed_bit_identical():
    h = host_layer("decode64", 8)
    c = h["cfg"]
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    idx, _ = oracle.select(oracle.router_logits(h["x"], h["router_w"], h["bias"]), c.k)
    res = []
    for packed in (False, True):
        blob = dev_packed("decode64") if packed else dev_weights("decode64")["blob"]
        y, a = moe.expert_ffn(to_dev(hl), blob, to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E, want_a=True,
                              packed=packed)
        res.append((from_dev(y), from_dev(a)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("T,d,L,F,E,k", [(3, 256, 384, 256, 100, 5), (2, 128, 128, 384, 8, 8)])
def test_layer_packed_ragged_scale_tiles(T, d, L, F, E, k):
    """K/128 not a multiple of 4: the last scale tile of a group is padded."""
    s = 0x5EED + 7 * T
    x = synth.normal_bf16(s, 1, 1.0, (T, d))
    Wr = synth.normal_bf16(s, 2, 0.02, (E, d))
    Wd = synth.normal_bf16(s, 3, 0.02, (L, d))
    Wu = synth.normal_bf16(s, 4, 0.02, (d, L))
    blob = synth.expert_blob(s, L, F, E)
    db = to_dev(blob)
    outs = [from_dev(moe.layer_forward(to_dev(x), to_dev(Wr), to_dev(Wd), to_dev(Wu),
                                       moe.pack_experts(db, E, L, F) if packed else db, k, d_ffn=F, packed=packed))
            for packed in (False, True)]
    assert np.array_equal(outs[0], outs[1])
    ref = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F)
    assert rel_l2(bf16_bits_to_f64(outs[1]), bf16_bits_to_f64(ref["out"])) <= 2e-3
