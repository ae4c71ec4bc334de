"""ctypes binding of the C oracle (moe_ref.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it to check and to time the GPU library.  Nothing in the
GPU library imports, links or calls it, and it shares no code with it.

bf16 tensors travel as numpy uint16 bit patterns.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_ref.c")
_LIB = os.path.join(_HERE, "libmoe_ref.so")

OK, ERR_ARG, ERR_UNSUPPORTED = 0, -1, -2
ACT_SILU, ACT_SITU = 0, 1
ACT_BF16, ACT_MXFP8 = 0, 1  # activation format at the expert GEMM inputs


def build() -> str:
    """Compile libmoe_ref.so: plain C99, one thread, no contraction of a*b+c."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.moe_ref_expert_bytes.argtypes = [i32, i32]
        L.moe_ref_expert_bytes.restype = ctypes.c_size_t
        L.moe_ref_e2m1.argtypes = [i32]
        L.moe_ref_e2m1.restype = ctypes.c_float
        L.moe_ref_mxfp4_value.argtypes = [i32, i32]
        L.moe_ref_mxfp4_value.restype = ctypes.c_float
        L.moe_ref_dequant_matrix.argtypes = [vp, vp, i64, i64, vp]
        L.moe_ref_bf16_from_f64.argtypes = [ctypes.c_double]
        L.moe_ref_bf16_from_f64.restype = ctypes.c_uint16
        L.moe_ref_dot_bf16_exact.argtypes = [vp, vp, i64]
        L.moe_ref_dot_bf16_exact.restype = ctypes.c_float
        L.moe_ref_router_logits.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
        L.moe_ref_select.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        L.moe_ref_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.moe_ref_linear_bf16.argtypes = [vp, vp, i64, i32, i32, vp]
        L.moe_ref_silu.argtypes = [ctypes.c_double]
        L.moe_ref_silu.restype = ctypes.c_double
        L.moe_ref_expert.argtypes = [vp, vp, i32, i32, i32, vp, vp]
        L.moe_ref_expert_fmt.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
        L.moe_ref_e4m3_value.argtypes = [i32]
        L.moe_ref_e4m3_value.restype = ctypes.c_double
        L.moe_ref_mxfp8_block.argtypes = [vp, vp, vp]
        L.moe_ref_layer_forward_fmt.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp,
                                                vp, vp, vp, i64, vp, vp, vp, vp, vp, vp]
        L.moe_ref_layer_forward_shared.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp,
                                                   vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, i32, i32]
        L.moe_ref_combine.argtypes = [vp, vp, i64, i32, i32, vp]
        L.moe_ref_reap_saliency.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp]
        L.moe_ref_layer_forward.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp,
                                            vp, vp, vp, i64, vp, vp, vp, vp, vp, vp]
        for name in ("moe_ref_dequant_matrix", "moe_ref_router_logits", "moe_ref_select",
                     "moe_ref_permute", "moe_ref_linear_bf16", "moe_ref_expert", "moe_ref_combine",
                     "moe_ref_layer_forward", "moe_ref_expert_fmt", "moe_ref_mxfp8_block",
                     "moe_ref_layer_forward_fmt", "moe_ref_reap_saliency", "moe_ref_layer_forward_shared"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != OK:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def expert_bytes(d_latent: int, d_ffn: int) -> int:
    return int(lib().moe_ref_expert_bytes(d_latent, d_ffn))


def e2m1(code: int) -> float:
    return float(lib().moe_ref_e2m1(code))


def mxfp4_value(code: int, scale: int) -> float:
    return float(lib().moe_ref_mxfp4_value(code, scale))


def dequant_matrix(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    _check(lib().moe_ref_dequant_matrix(_p(codes), _p(scales), rows, cols, _p(out)), "dequant")
    return out


def expert_matrices(record: np.ndarray, d_latent: int, d_ffn: int):
    """Split one expert record into (gate, up, down) fp32 matrices."""
    L, F = d_latent, d_ffn
    mat = F * L // 2 + F * L // 32
    g = dequant_matrix(np.ascontiguousarray(record[0:F * L // 2]),
                       np.ascontiguousarray(record[F * L // 2:mat]), F, L)
    u = dequant_matrix(np.ascontiguousarray(record[mat:mat + F * L // 2]),
                       np.ascontiguousarray(record[mat + F * L // 2:2 * mat]), F, L)
    dn = dequant_matrix(np.ascontiguousarray(record[2 * mat:2 * mat + L * F // 2]),
                        np.ascontiguousarray(record[2 * mat + L * F // 2:3 * mat]), L, F)
    return g, u, dn


def bf16_from_f64(v: float) -> int:
    return int(lib().moe_ref_bf16_from_f64(float(v)))


def dot_bf16_exact(a: np.ndarray, b: np.ndarray) -> float:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    assert a.size == b.size
    return float(lib().moe_ref_dot_bf16_exact(_p(a), _p(b), a.size))


def _spans(n: int, threads: int):
    """[lo, hi) token ranges for up to `threads` shards of n tokens."""
    parts = max(1, min(threads, n))
    cuts = [n * i // parts for i in range(parts + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(parts) if cuts[i + 1] > cuts[i]]


def _run_shards(fn, spans):
    """Run fn(lo, hi) for every span, in threads when there are several: the C library
    keeps no state between calls and ctypes releases the GIL during each call, so the
    shards run in parallel; each shard is the single-threaded oracle on its tokens."""
    if len(spans) <= 1:
        return [fn(lo, hi) for lo, hi in spans]
    with cf.ThreadPoolExecutor(len(spans)) as ex:
        return list(ex.map(lambda s: fn(*s), spans))


def router_logits(x: np.ndarray, router_w: np.ndarray, bias: Optional[np.ndarray] = None,
                  threads: int = 1) -> np.ndarray:
    T, d = x.shape
    E = router_w.shape[0]
    bias_stride = 0 if bias is None or bias.ndim == 1 else E
    out = np.empty((T, E), dtype=np.float32)

    def shard(lo, hi):
        b = None if bias is None else (bias if bias_stride == 0 else bias[lo:hi])
        _check(lib().moe_ref_router_logits(_p(x[lo:hi]), _p(router_w), _p(b), bias_stride, hi - lo, d, E,
                                           _p(out[lo:hi])), "router_logits")

    _run_shards(shard, _spans(T, threads))
    return out


def select(logits: np.ndarray, k: int, renormalize: bool = True, threads: int = 1):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)

    def shard(lo, hi):
        _check(lib().moe_ref_select(_p(logits[lo:hi]), hi - lo, E, k, int(renormalize), _p(idx[lo:hi]),
                                    _p(w[lo:hi])), "select")

    _run_shards(shard, _spans(T, threads))
    return idx, w


def permute(idx: np.ndarray, num_experts: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(num_experts, dtype=np.int32)
    offsets = np.empty(num_experts + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    _check(lib().moe_ref_permute(_p(idx), T, k, num_experts, _p(counts), _p(offsets), _p(perm)), "permute")
    return counts, offsets, perm


def linear_bf16(inp: np.ndarray, W: np.ndarray) -> np.ndarray:
    T, n_in = inp.shape
    n_out = W.shape[0]
    out = np.empty((T, n_out), dtype=np.uint16)
    _check(lib().moe_ref_linear_bf16(_p(inp), _p(W), T, n_in, n_out, _p(out)), "linear")
    return out


def silu(g: float) -> float:
    return float(lib().moe_ref_silu(float(g)))


def e4m3_value(code: int) -> float:
    return float(lib().moe_ref_e4m3_value(code))


def mxfp8_block(v) -> tuple:
    """MXFP8 of 32 values (OCP MX convention): (codes uint8 [32], e8m0 scale byte)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    assert v.shape == (32,)
    codes = np.empty(32, dtype=np.uint8)
    sc = np.empty(1, dtype=np.uint8)
    _check(lib().moe_ref_mxfp8_block(_p(v), _p(codes), _p(sc)), "mxfp8_block")
    return codes, int(sc[0])


def expert(h: np.ndarray, record: np.ndarray, d_latent: int, d_ffn: int, act: int = ACT_SILU,
           act_format: int = ACT_BF16):
    """One expert on one latent row: returns (a bf16 bits [F], y fp32 [L])."""
    a = np.empty(d_ffn, dtype=np.uint16)
    y = np.empty(d_latent, dtype=np.float32)
    _check(lib().moe_ref_expert_fmt(_p(np.ascontiguousarray(h)), _p(np.ascontiguousarray(record)), d_latent,
                                    d_ffn, act, act_format, _p(a), _p(y)), "expert")
    return a, y


def reap_saliency(y: np.ndarray, w: np.ndarray, idx: np.ndarray, num_experts: int) -> np.ndarray:
    """Sum over routed rows of w * ||y||_2 per expert (fp64 [E]); y [T*k, L] by slot."""
    T, k = idx.shape
    s = np.zeros(num_experts, dtype=np.float64)
    _check(lib().moe_ref_reap_saliency(_p(np.ascontiguousarray(y, dtype=np.float32)),
                                       _p(np.ascontiguousarray(w, dtype=np.float32)),
                                       _p(np.ascontiguousarray(idx, dtype=np.int32)), T, k, y.shape[1],
                                       num_experts, _p(s)), "reap_saliency")
    return s


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y fp32 [T*k, L] in slot order, w fp32 [T, k] -> z bf16 bits [T, L]."""
    T, k = w.shape
    L = y.shape[1]
    z = np.empty((T, L), dtype=np.uint16)
    _check(lib().moe_ref_combine(_p(np.ascontiguousarray(y)), _p(np.ascontiguousarray(w)), T, k, L, _p(z)),
           "combine")
    return z


def layer_forward(x, router_w, latent_down, latent_up, blob, k: int, d_latent: int, d_ffn: int,
                  bias: Optional[np.ndarray] = None, tokens: Optional[Sequence[int]] = None,
                  act: int = ACT_SILU, renormalize: bool = True, act_format: int = ACT_BF16,
                  shared_blob: Optional[np.ndarray] = None, num_shared: int = 0, d_ffn_shared: int = 0,
                  threads: int = 1) -> dict:
    """Whole layer for `tokens` (default: all).  Returns dict of out, idx, w, logits, h, z.
    threads > 1 splits the tokens into shards computed side by side (tokens are
    independent in the layer, so the result is the same)."""
    T, d = x.shape
    E = router_w.shape[0]
    bias_stride = 0 if bias is None or bias.ndim == 1 else E
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, dtype=np.int32)
    n = tok.size
    out = np.empty((n, d), dtype=np.uint16)
    idx = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float32)
    logits = np.empty((n, E), dtype=np.float32)
    h = np.empty((n, d_latent), dtype=np.uint16)
    z = np.empty((n, d_latent), dtype=np.uint16)
    sb = None if shared_blob is None else np.ascontiguousarray(shared_blob)

    def shard(lo, hi):
        t = np.ascontiguousarray(tok[lo:hi])
        rc = lib().moe_ref_layer_forward_shared(d, d_latent, d_ffn, E, k, act, act_format, int(renormalize), _p(x),
                                                _p(router_w), _p(bias), bias_stride, _p(latent_down), _p(latent_up),
                                                _p(blob), _p(t), hi - lo, _p(out[lo:hi]), _p(idx[lo:hi]),
                                                _p(w[lo:hi]), _p(logits[lo:hi]), _p(h[lo:hi]), _p(z[lo:hi]),
                                                _p(sb), num_shared, d_ffn_shared)
        _check(rc, "layer_forward")

    _run_shards(shard, _spans(n, threads))
    return dict(out=out, idx=idx, w=w, logits=logits, h=h, z=z)
