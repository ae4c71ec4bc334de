"""Parity of the HIP library (through its C ABI) with the CPU oracle.

Bit-exact: MXFP4 dequantisation, top-k selection on shared logits, the exact
routing of every token, and the permutation.  Floating-point layer outputs:
relative L2 error <= 2e-3 (fp32 accumulation, bf16 in/out).
"""
import math

import numpy as np
import pytest
import torch

import mxfp4_expert_gemm_amd as moe
import oracle
import synth
from _util import bf16_bits_to_f64, f64_to_bf16_bits, rel_l2
from gpu_common import ORACLE_THREADS, dev_weights, from_dev, host_layer, log, oracle_routing, to_dev

pytestmark = pytest.mark.gpu

TOL_OUT = 2e-3


def _same_f32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return ((a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))).all()


# ----------------------------------------------------------------- dequant

def test_dequant_every_code_and_scale():
    """256 rows, one per e8m0 value; each row holds every byte value once (all 16x16 code pairs)."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 256)
    scales = np.repeat(np.arange(256, dtype=np.uint8), 16)
    got = from_dev(moe.dequant_mxfp4(to_dev(codes), to_dev(scales), 256, 512))
    want = oracle.dequant_matrix(codes, scales, 256, 512)
    assert _same_f32(got, want)


def test_dequant_k3_records_bit_exact():
    h = host_layer("decode1")
    blob = h["blob"]
    dblob = dev_weights("decode1")["blob"]
    L, F = 3584, 3072
    rec = synth.expert_record_bytes(L, F)
    nc, mat = F * L // 2, F * L // 2 + F * L // 32
    for e in (0, 447, 895):
        for m, (rows, cols) in enumerate([(F, L), (F, L), (L, F)]):
            base = e * rec + m * mat
            got = from_dev(moe.dequant_mxfp4(dblob[base:base + nc], dblob[base + nc:base + mat], rows, cols))
            want = oracle.dequant_matrix(blob[base:base + nc], blob[base + nc:base + mat], rows, cols)
            assert _same_f32(got, want), (e, m)


# ------------------------------------------------------------------- top-k

@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (8, 8), (100, 7), (896, 16), (1024, 64)])
def test_topk_on_shared_logits_bit_exact(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 300
    pool = np.array([-1.0, 0.0, -0.0, 1.0, 2.0, np.nan, -np.inf, np.inf, 0.5], dtype=np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[: T // 2] = pool[rng.integers(0, pool.size, (T // 2, E))]
    idx, w = moe.topk(to_dev(logits), k)
    want_idx, want_w = oracle.select(logits, k)
    assert np.array_equal(from_dev(idx), want_idx)
    gw = from_dev(w)
    fin = np.isfinite(want_w)
    assert np.allclose(gw[fin], want_w[fin], rtol=2e-6, atol=1e-7)


# ----------------------------------------------------------------- routing

def test_route_tiny_every_logit_exact():
    h = host_layer("tiny")
    dw = dev_weights("tiny")
    c = h["cfg"]
    logits, idx, w = moe.route(to_dev(h["x"]), dw["router_w"], c.k, flags=moe.ROUTE_EXACT_ALL)
    want = oracle.router_logits(h["x"], h["router_w"])
    assert _same_f32(from_dev(logits), want)
    want_idx, want_w = oracle.select(want, c.k)
    assert np.array_equal(from_dev(idx), want_idx)
    assert np.allclose(from_dev(w), want_w, rtol=2e-6, atol=0)


def _bf(v):
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


def test_route_exact_path_decides_midpoints():
    """Rows whose exact logits sit on or next to an fp32 rounding midpoint: only the
    fixed-point accumulator can round them; the oracle's exact dot must agree."""
    d, E = 64, 8
    x = np.zeros((4, d), np.uint16)
    W = np.zeros((E, d), np.uint16)
    one, tiny, far = _bf(1.0), _bf(2.0 ** -12), _bf(2.0 ** -60)
    x[:, 0], x[:, 1] = one, tiny
    x[1, 2] = far
    x[2, 2] = _bf(-(2.0 ** -60))
    x[3, 3] = _bf(3.0)
    for e in range(E):
        W[e, 0], W[e, 1] = one, tiny
        W[e, 2] = far
        W[e, 3] = _bf(2.0 ** (-70 - e))
    logits, idx, w = moe.route(to_dev(x), to_dev(W), 3, flags=moe.ROUTE_EXACT_ALL)
    want = oracle.router_logits(x, W)
    assert _same_f32(from_dev(logits), want)
    assert np.array_equal(from_dev(idx), oracle.select(want, 3)[0])


@pytest.mark.parametrize("name", ["tiny", "decode1", "decode64", "prefill4k", "prefill32k"])
def test_route_indices_bit_exact(name):
    """Every token of every workload: the GPU's certified routing selects exactly the
    oracle's experts (the correctly rounded logits' top-k, lowest index on ties)."""
    h = host_layer(name)
    c = h["cfg"]
    dw = dev_weights(name)
    bias = None if h["bias"] is None else to_dev(h["bias"])
    log(f"route {name} T={h['x'].shape[0]}")
    logits, idx, w = moe.route(to_dev(h["x"]), dw["router_w"], c.k, bias=bias)
    want_l, want_idx, want_w = oracle_routing(name)
    gidx = from_dev(idx)
    bad = np.nonzero((gidx != want_idx).any(1))[0]
    assert bad.size == 0, f"{bad.size} tokens routed differently, first {bad[:8].tolist()}"
    gl = from_dev(logits).astype(np.float64)
    dev_max = np.max(np.abs(gl - want_l))
    log(f"  max |logit - exact| = {dev_max:.3g}")
    assert dev_max < 1e-3
    assert np.allclose(from_dev(w), want_w, rtol=1e-4, atol=1e-6)


def test_route_batch_builds_agree():
    """Batches of 2048 tokens and more route on a build capped at 128 registers a lane,
    smaller ones on the uncapped build: 2048 and 2047 tokens of prefill4k route their
    common tokens identically (indices, weights and logits bit for bit)."""
    h = host_layer("prefill4k")
    c = h["cfg"]
    dw = dev_weights("prefill4k")
    xs = h["x"][:2048]
    bias = h["bias"]

    def run(T):
        b = None if bias is None else to_dev(bias[:T] if bias.ndim == 2 else bias)
        return [from_dev(t) for t in moe.route(to_dev(xs[:T]), dw["router_w"], c.k, bias=b)]

    big, small = run(2048), run(2047)
    for a, b in zip(big, small):
        assert np.array_equal(a[:2047].view(np.uint32) if a.dtype == np.float32 else a[:2047],
                              b.view(np.uint32) if b.dtype == np.float32 else b)


@pytest.mark.parametrize("T", [3, 40, 300])
def test_route_subnormal_inputs_recomputed(T):
    """Tokens and router rows holding subnormal bf16 values (which the matrix cores or
    dot instructions may flush) are routed exactly: their norms are +inf, so every
    logit that can matter is recomputed.  T = 3 takes the GEMV, 40 and 300 the GEMM."""
    d, E, k = 256, 64, 6
    x = synth.normal_bf16(77 + T, 1, 1.0, (T, d))
    W = synth.normal_bf16(77 + T, 2, 0.05, (E, d))
    x[0, 5] = 0x0001             # smallest positive subnormal
    x[T - 1, d - 1] = 0x807F     # largest negative subnormal
    W[9, 17] = 0x0040
    logits, idx, w = moe.route(to_dev(x), to_dev(W), k)
    want_l = oracle.router_logits(x, W)
    want_idx, _ = oracle.select(want_l, k)
    assert np.array_equal(from_dev(idx), want_idx)
    assert np.max(np.abs(from_dev(logits).astype(np.float64) - want_l)) < 1e-3


# ------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,k,E", [(1, 16, 896), (16, 2, 8), (64, 16, 896), (3, 5, 100), (4096, 16, 896),
                                   (32768, 16, 896)])
def test_permute_bit_exact(T, k, E):
    rng = np.random.default_rng(T + k + E)
    p = rng.random(E) ** 3
    p /= p.sum()
    idx = np.stack([np.sort(rng.choice(E, k, replace=False, p=p)) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = moe.permute(to_dev(idx), E)
    wc, wo, wp = oracle.permute(idx, E)
    assert np.array_equal(from_dev(counts), wc)
    assert np.array_equal(from_dev(offsets), wo)
    assert np.array_equal(from_dev(perm), wp)


# --------------------------------------------------------- dense + experts

@pytest.mark.parametrize("T,n_in,n_out", [(1, 7168, 3584), (3, 3584, 7168), (16, 256, 128), (5, 128, 96),
                                          # matrix-core GEMM: ragged token and row tiles, fewer K tiles
                                          # than are prefetched, both tile shapes
                                          (33, 64, 16), (40, 256, 96), (257, 192, 200), (512, 7168, 3584)])
def test_linear_bf16(T, n_in, n_out):
    a = synth.normal_bf16(5, 1, 1.0, (T, n_in))
    W = synth.normal_bf16(5, 2, 0.02, (n_out, n_in))
    got = from_dev(moe.linear_bf16(to_dev(a), to_dev(W)))
    want = oracle.linear_bf16(a, W)
    assert rel_l2(bf16_bits_to_f64(got), bf16_bits_to_f64(want)) < 1e-4
    assert np.mean(got == want) > 0.99


@pytest.mark.parametrize("n_in,n_out", [(7168, 3584), (3584, 7168)])
def test_linear_bf16_kernel_choice(n_in, n_out):
    """4133 tokens in 128 x 128 tiles make a grid of 924 or 1848 blocks, which runs the
    LDS-direct matrix-core kernel; their first 256 tokens alone make 56 or 112 blocks, under
    the 768 it needs, and run the register-staged one.  Both take the same K-tile arithmetic,
    so the shared rows agree bit for bit; the ragged last tile matches the oracle."""
    a = synth.normal_bf16(7, 1, 1.0, (4096 + 37, n_in))
    W = synth.normal_bf16(7, 2, 0.02, (n_out, n_in))
    dW = to_dev(W)
    big = from_dev(moe.linear_bf16(to_dev(a), dW))
    small = from_dev(moe.linear_bf16(to_dev(a[:256]), dW))
    assert np.array_equal(big[:256], small)
    want = oracle.linear_bf16(a[-37:], W)
    assert rel_l2(bf16_bits_to_f64(big[-37:]), bf16_bits_to_f64(want)) < 1e-4


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode1", None), ("decode64", 8)])
def test_expert_ffn(name, T):
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    Tn = h["x"].shape[0]
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    lg = oracle.router_logits(h["x"], h["router_w"], h["bias"])
    idx, w = oracle.select(lg, c.k)
    y, a = moe.expert_ffn(to_dev(hl), dw["blob"], to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E,
                          want_a=True)
    y, a = from_dev(y), from_dev(a)
    rec = c.record_bytes
    ulps, yerr = [], []
    for t in range(Tn):
        for j in range(c.k):
            e = int(idx[t, j])
            wa, wy = oracle.expert(hl[t], h["blob"][e * rec:(e + 1) * rec], c.L, c.F)
            r = t * c.k + j
            # same-sign bf16 patterns are ordered like the values they encode
            ulps.append(np.abs(a[r].astype(np.int64) - wa.astype(np.int64)))
            yerr.append(rel_l2(y[r], wy))
    ulps = np.concatenate(ulps)
    log(f"  a: exact {np.mean(ulps == 0):.4f}, within 1 ulp {np.mean(ulps <= 1):.5f}; "
        f"y rel-L2 max {max(yerr):.3g} mean {np.mean(yerr):.3g}")
    # a is bf16 of silu(g) u with g, u summed on the matrix cores (about 2^-22 of the sum of
    # |products| per 128-product instruction) and exactly by the oracle: where the two
    # straddle a rounding boundary a moves by an ulp (a few ulps where g or u cancel to a
    # tiny value), which moves y by about 2^-8 sqrt(flip fraction) relative
    assert np.mean(ulps == 0) > 0.95 and np.mean(ulps <= 1) > 0.99
    assert max(yerr) < 1e-3


def test_expert_ffn_grouped_gemm_and_streaming_kernels_against_the_oracle():
    """The same routed rows through the streaming kernels (32 rows) and the grouped GEMMs
    (96 rows: at least 8 per expert on average): the two run different matrix-core shapes
    (16x16x128 against 32x32x64), so their fp32 sums differ in order; every row of both is
    checked against the oracle, and the rows they share agree to the same tolerance."""
    c = synth.CONFIGS["tiny"]
    h = host_layer("tiny")
    dw = dev_weights("tiny")
    x = synth.make_tokens(c, T=48)
    hl = oracle.linear_bf16(x, h["latent_down"])
    idx, _ = oracle.select(oracle.router_logits(x, h["router_w"], None), c.k)
    small = moe.expert_ffn(to_dev(hl[:16]), dw["blob"], to_dev(idx[:16]), d_model=c.d, d_ffn=c.F, num_experts=c.E,
                           want_a=True)   # 32 rows: streaming kernels
    big = moe.expert_ffn(to_dev(hl), dw["blob"], to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E,
                         want_a=True)     # 96 rows: grouped GEMMs
    ys, as_ = from_dev(small[0]), from_dev(small[1])
    yb, ab = from_dev(big[0]), from_dev(big[1])
    rec = c.record_bytes
    ulps = []
    for t in range(48):
        for j in range(c.k):
            e, r = int(idx[t, j]), t * c.k + j
            wa, wy = oracle.expert(hl[t], h["blob"][e * rec:(e + 1) * rec], c.L, c.F)
            assert rel_l2(yb[r], wy) < 1e-3, (t, j)
            ulps.append(np.abs(ab[r].astype(np.int64) - wa.astype(np.int64)))
            if t < 16:
                assert rel_l2(ys[r], wy) < 1e-3, (t, j)
                assert rel_l2(yb[r], ys[r]) < 1e-3, (t, j)
    ulps = np.concatenate(ulps)
    assert np.mean(ulps == 0) > 0.95 and np.mean(ulps <= 1) > 0.99


@pytest.mark.parametrize("name,idx_rows", [
    ("tiny", [[5, 5], [5, 1], [5, 5]]),       # expert 5 takes 5 rows, 3 of one token: two passes
    ("decode1", [[7] * 16]),                  # one token, one expert in all 16 slots: four passes
])
def test_expert_ffn_repeated_experts(name, idx_rows):
    """A caller may give an expert several slots of one token (the router never does): every
    slot is still its own row, with the same bits as that (token, expert) pair computed
    alone, and within the oracle's tolerance."""
    h = host_layer(name, len(idx_rows))
    c = h["cfg"]
    dw = dev_weights(name)
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    idx = np.array(idx_rows, dtype=np.int32)
    T, k = idx.shape
    y, a = moe.expert_ffn(to_dev(hl), dw["blob"], to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E,
                          want_a=True)
    y, a = from_dev(y), from_dev(a)
    rec = c.record_bytes
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            # the pair alone: token t with e in slot 0 and distinct other experts
            others = [x for x in range(c.E) if x != e][:k - 1]
            one = np.array([[e] + others], dtype=np.int32)
            y1, a1 = moe.expert_ffn(to_dev(hl[t:t + 1]), dw["blob"], to_dev(one), d_model=c.d, d_ffn=c.F,
                                    num_experts=c.E, want_a=True)
            r = t * k + j
            assert np.array_equal(y[r], from_dev(y1)[0]) and np.array_equal(a[r], from_dev(a1)[0]), (t, j)
            if j == 0 or idx[t, j] != idx[t, 0]:
                _, wy = oracle.expert(hl[t], h["blob"][e * rec:(e + 1) * rec], c.L, c.F)
                assert rel_l2(y[r], wy) < 1e-3


def test_expert_ffn_skips_ids_out_of_range():
    """Slots whose expert id lies outside [0, E) are skipped: their rows of y and a keep
    what the caller's buffers held; every other slot is its pair computed alone."""
    name = "tiny"
    idx = np.array([[2, -1], [8, 3], [1, 100]], dtype=np.int32)
    h = host_layer(name, idx.shape[0])
    c = h["cfg"]
    dw = dev_weights(name)
    hl = oracle.linear_bf16(h["x"], h["latent_down"])
    T, k = idx.shape
    y = torch.full((T * k, c.L), float("nan"), dtype=torch.float32, device="cuda")
    a = torch.full((T * k, c.F), 0x7E5A, dtype=torch.int16, device="cuda")
    moe.expert_ffn(to_dev(hl), dw["blob"], to_dev(idx), d_model=c.d, d_ffn=c.F, num_experts=c.E, y=y, a=a)
    y, a = from_dev(y), from_dev(a)
    for t in range(T):
        for j in range(k):
            e, r = int(idx[t, j]), t * k + j
            if not 0 <= e < c.E:
                assert np.isnan(y[r]).all() and (a[r] == 0x7E5A).all(), (t, j)
                continue
            one = np.array([[e] + [x for x in range(c.E) if x != e][:k - 1]], dtype=np.int32)
            y1, a1 = moe.expert_ffn(to_dev(hl[t:t + 1]), dw["blob"], to_dev(one), d_model=c.d, d_ffn=c.F,
                                    num_experts=c.E, want_a=True)
            assert np.array_equal(y[r], from_dev(y1)[0]) and np.array_equal(a[r], from_dev(a1)[0]), (t, j)


def test_combine():
    rng = np.random.default_rng(1)
    T, k, L = 33, 16, 3584
    y = rng.standard_normal((T * k, L)).astype(np.float32) * 1e3
    _, w = oracle.select(rng.standard_normal((T, 896)).astype(np.float32), k)
    got = from_dev(moe.combine(to_dev(y), to_dev(w), dtype=torch.int16))
    want = oracle.combine(y, w)
    # fp32 accumulation of k terms vs fp64: per element the difference stays within one bf16
    # rounding of the result plus k fp32 roundings of partial sums bounded by sum_j |w_j y_j|
    g, r = bf16_bits_to_f64(got), bf16_bits_to_f64(want)
    mag = np.einsum("tj,tjl->tl", np.abs(w).astype(np.float64), np.abs(y.reshape(T, k, L)).astype(np.float64))
    # |RN(a) - RN(b)| <= |a - b| + one ulp (each rounding moves by at most half an ulp <= 2^-8 |value|)
    assert (np.abs(g - r) <= 2.0 ** -7 * np.maximum(np.abs(g), np.abs(r)) + k * 2.0 ** -23 * mag).all()
    assert np.mean(got == want) > 0.999


def test_combine_past_65535_tokens():
    """More tokens than a grid's second dimension could hold (the combine grid is flat
    over tokens x latent quads): every token, the last ones included, as the oracle's
    fp64 combine."""
    rng = np.random.default_rng(2)
    T, k, L = 70001, 2, 128
    y = rng.standard_normal((T * k, L)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    got = from_dev(moe.combine(to_dev(y), to_dev(w), dtype=torch.int16))
    want = oracle.combine(y, w)
    assert np.array_equal(got[65530:], want[65530:])
    assert np.mean(got == want) > 0.999


def test_combine_grid_stride_pass():
    """The flat combine grid is capped at 2^20 blocks of 256 threads (2^28 quads of latent
    values); a batch past that takes a second grid-stride pass.  First tokens and the
    tail (second pass) against the oracle's fp64 combine."""
    T, k, L = (1 << 25) + 4099, 1, 32
    g = torch.Generator(device="cuda").manual_seed(3)
    y = torch.randn(T * k, L, device="cuda", generator=g)
    w = torch.rand(T, k, device="cuda", generator=g)
    z = moe.combine(y, w, dtype=torch.int16)
    rows = torch.cat([torch.arange(0, 64), torch.arange(T - 8192, T)]).cuda()
    got = from_dev(z[rows])
    want = oracle.combine(from_dev(y[rows]), from_dev(w[rows]))
    assert np.array_equal(got, want)


# ------------------------------------------------------------- whole layer

def _layer_case(name, T=None, sample=None):
    """The layer on a workload: routing, grouping and counts of every token against the
    oracle's (bit-exact), outputs against the oracle's on `sample` (default: every token)
    to the relative L2 tolerance.  Returns the outputs and routing outputs."""
    h = host_layer(name, T)
    c = h["cfg"]
    dw = dev_weights(name)
    Tn = h["x"].shape[0]
    x = to_dev(h["x"])
    bias = None if h["bias"] is None else to_dev(h["bias"])
    routing = dict(topk_idx=torch.empty((Tn, c.k), dtype=torch.int32, device="cuda"),
                   topk_w=torch.empty((Tn, c.k), dtype=torch.float32, device="cuda"),
                   logits=torch.empty((Tn, c.E), dtype=torch.float32, device="cuda"),
                   expert_counts=torch.empty(c.E, dtype=torch.int32, device="cuda"),
                   expert_offsets=torch.empty(c.E + 1, dtype=torch.int32, device="cuda"),
                   perm=torch.empty(Tn * c.k, dtype=torch.int32, device="cuda"))
    log(f"layer {name} T={Tn}")
    out = moe.layer_forward(x, dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k, d_ffn=c.F,
                            bias=bias, routing=routing)
    torch.cuda.synchronize()
    out = from_dev(out)
    got = {k: from_dev(v) for k, v in routing.items()}
    gidx = got["topk_idx"]
    tokens = list(range(Tn)) if sample is None else sorted(set(sample))
    ref = oracle.layer_forward(h["x"], h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F,
                               bias=h["bias"], tokens=tokens, threads=ORACLE_THREADS)
    assert np.array_equal(gidx[tokens], ref["idx"])
    if T is None:
        # every token's experts and weights, against the oracle's routing of the whole batch
        _, want_idx, want_w = oracle_routing(name)
        assert np.array_equal(gidx, want_idx)
        assert np.allclose(got["topk_w"], want_w, rtol=1e-4, atol=1e-6)
    err = rel_l2(bf16_bits_to_f64(out[tokens]), bf16_bits_to_f64(ref["out"]))
    log(f"  rel-L2 over {len(tokens)} tokens = {err:.3g}")
    assert err <= TOL_OUT
    # the grouping: the oracle's grouping of the (oracle-equal) routing
    wc, wo, wp = oracle.permute(gidx, c.E)
    assert np.array_equal(got["expert_counts"], wc)
    assert np.array_equal(got["expert_offsets"], wo)
    assert np.array_equal(got["perm"], wp)
    assert (wc.sum() == Tn * c.k) and all(len(set(r)) == c.k for r in gidx.tolist())
    return out, got


def test_layer_tiny():
    _layer_case("tiny")


def test_layer_tiny_past_65535_tokens():
    """70001 tokens: more than a grid's second dimension holds; outputs of tokens on both
    sides of 65535 against the oracle, routing and grouping of every token checked."""
    out, got = _layer_case("tiny", T=70001, sample=[0, 65534, 65535, 65536, 70000])
    h = host_layer("tiny", 70001)
    assert h["bias"] is None
    ridx = oracle.select(oracle.router_logits(h["x"], h["router_w"], None, threads=ORACLE_THREADS), h["cfg"].k)[0]
    assert np.array_equal(got["topk_idx"], ridx)


def test_layer_decode1():
    _layer_case("decode1")


def test_layer_decode64_every_token():
    _layer_case("decode64")


def test_layer_prefill4k_full_size():
    """All 4096 tokens through the layer: routing, weights and grouping of every token
    against the oracle's; outputs on a seeded sample (first, last and spread)."""
    rng = np.random.default_rng(0x4096)
    _layer_case("prefill4k", sample=[0, 4095] + rng.choice(4096, 30, replace=False).tolist())


def test_layer_prefill32k_full_size():
    rng = np.random.default_rng(0x32768)
    _layer_case("prefill32k", sample=[0, 32767] + rng.choice(32768, 30, replace=False).tolist())


def test_layer_prefill4k_run_twice_bit_identical():
    """The prefill path (integer atomics in the grouping, grouped GEMMs, the combine) gives
    the same bits on a second run: outputs, routing, grouping."""
    h = host_layer("prefill4k")
    c = h["cfg"]
    dw = dev_weights("prefill4k")
    runs = []
    for _ in range(2):
        routing = dict(topk_idx=torch.empty((c.T, c.k), dtype=torch.int32, device="cuda"),
                       topk_w=torch.empty((c.T, c.k), dtype=torch.float32, device="cuda"),
                       expert_offsets=torch.empty(c.E + 1, dtype=torch.int32, device="cuda"),
                       perm=torch.empty(c.T * c.k, dtype=torch.int32, device="cuda"))
        out = moe.layer_forward(to_dev(h["x"]), dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k,
                                d_ffn=c.F, bias=to_dev(h["bias"]), routing=routing)
        torch.cuda.synchronize()
        runs.append([from_dev(out)] + [from_dev(v) for v in routing.values()])
    for a, b in zip(*runs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("T", [40, 600, 1100])
def test_layer_tiny_weights_every_dispatch_path(T):
    """T*k of 80, 1200 and 2200 rows: the unfused down + combine kernels, the routing kernel
    without the fused permutation, and the chunked permutation."""
    c = synth.CONFIGS["tiny"]
    h = host_layer("tiny")
    dw = dev_weights("tiny")
    x = synth.make_tokens(c, T=T)
    idx = torch.empty((T, c.k), dtype=torch.int32, device="cuda")
    out = moe.layer_forward(to_dev(x), dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k,
                            d_ffn=c.F, routing={"topk_idx": idx})
    ref = oracle.layer_forward(x, h["router_w"], h["latent_down"], h["latent_up"], h["blob"], c.k, c.L, c.F)
    assert np.array_equal(from_dev(idx), ref["idx"])
    assert rel_l2(bf16_bits_to_f64(from_dev(out)), bf16_bits_to_f64(ref["out"])) <= TOL_OUT


def test_layer_deterministic():
    a, _ = _layer_case("tiny")
    b, _ = _layer_case("tiny")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T,d,L,F,E,k", [(3, 256, 128, 256, 100, 5), (1, 128, 128, 128, 8, 8), (7, 64, 256, 128, 2, 1)])
def test_layer_ragged_shapes(T, d, L, F, E, k):
    s = 0x5EED + T
    x = synth.normal_bf16(s, 1, 1.0, (T, d))
    Wr = synth.normal_bf16(s, 2, 0.02, (E, d))
    Wd = synth.normal_bf16(s, 3, 0.02, (L, d))
    Wu = synth.normal_bf16(s, 4, 0.02, (d, L))
    blob = synth.expert_blob(s, L, F, E)
    out = moe.layer_forward(to_dev(x), to_dev(Wr), to_dev(Wd), to_dev(Wu), to_dev(blob), k, d_ffn=F)
    ref = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F)
    assert rel_l2(bf16_bits_to_f64(from_dev(out)), bf16_bits_to_f64(ref["out"])) <= TOL_OUT


@pytest.mark.parametrize("ndup", [12, 100])
def test_layer_one_token_repeated_router_rows(ndup):
    """One token (the block-wide routing kernel) whose ndup best router rows are copies of one
    row: equal logits straddle the top-8 boundary, which no error radius can certify, and
    with 100 copies there are more candidates than one wave ranks.  The selection is then
    decided exactly: the copies with the lowest indices."""
    T, d, L, F, E, k = 1, 256, 128, 128, 300, 8
    s = 0xD0B + ndup
    x = synth.normal_bf16(s, 1, 1.0, (T, d))
    Wr = synth.normal_bf16(s, 2, 0.02, (E, d))
    rows = synth.permutation(s, 3, E)[:ndup]
    # a row aligned with the token, far above the random rows, repeated ndup times
    Wr[rows] = np.where(bf16_bits_to_f64(x[0]) >= 0, 0x3CA4, 0xBCA4).astype(np.uint16)  # +-0.02
    Wd = synth.normal_bf16(s, 4, 0.02, (L, d))
    Wu = synth.normal_bf16(s, 5, 0.02, (d, L))
    blob = synth.expert_blob(s, L, F, E)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = moe.layer_forward(to_dev(x), to_dev(Wr), to_dev(Wd), to_dev(Wu), to_dev(blob), k, d_ffn=F,
                            routing={"topk_idx": idx})
    ref = oracle.layer_forward(x, Wr, Wd, Wu, blob, k, L, F)
    assert np.array_equal(ref["idx"][0], np.sort(rows)[:k])
    assert np.array_equal(from_dev(idx), ref["idx"])
    assert rel_l2(bf16_bits_to_f64(from_dev(out)), bf16_bits_to_f64(ref["out"])) <= TOL_OUT


def test_layer_zero_tokens_is_a_noop():
    dw = dev_weights("tiny")
    c = synth.CONFIGS["tiny"]
    x = torch.empty((0, c.d), dtype=torch.int16, device="cuda")
    out = moe.layer_forward(x, dw["router_w"], dw["latent_down"], dw["latent_up"], dw["blob"], c.k, d_ffn=c.F,
                            workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, c.d)
