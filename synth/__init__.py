"""Seeded synthetic inputs for the Stable-LatentMoE layer with MXFP4 experts.

This module holds only random-number generation and the shapes, layouts and
value distributions of the inputs: none of the layer's arithmetic.  The CPU
oracle (``oracle/``) and the GPU path (``mxfp4_expert_gemm_amd``) both take
their inputs from here, so they always see identical bytes.

The workloads mirror the shapes the pages describe for one Kimi-K3 MoE layer:
896 routed experts with top-16 routing (kimi-k3-mlx digest, architecture
table), a 3584-wide latent space under a 7168-wide residual (same table,
"Stable LatentMoE" row), and experts shipped as MXFP4 with one 8-bit exponent
per 32 weights, 17,547,264 bytes per expert (kimi-k3-in-c post, section on
experts that are already 4-bit MXFP4).  The prompt cap of 32,768 tokens comes
from the kimi-k3-in-c post's section on what the engine does not cover; the
domain-clustered routing of the largest workload mimics the digest's section
on experts clustering by domain.  No public dataset or checkpoint is used: the
real hidden states and weights are stood in for by the seeded draws below.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# stream ids: one independent counter-based stream per tensor
S_X, S_ROUTER, S_DOWN, S_UP, S_CODES, S_SCALES, S_ZIPF, S_DOMAIN, S_CLUSTER = range(1, 10)

SCALE_LO, SCALE_HI = 120, 130  # e8m0 exponents drawn uniformly in [120, 130]


def build() -> str:
    """Compile libsynth.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", _LIB + ".tmp", "-lm"]
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
        u64, i64, i32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_draw.argtypes = [u64, u64, u64]
        L.synth_draw.restype = u64
        L.synth_normal.argtypes = [u64, u64, u64]
        L.synth_normal.restype = f64
        L.synth_normal_bf16.argtypes = [u64, u64, f64, u64, i64, vp]
        L.synth_bytes.argtypes = [u64, u64, u64, i64, vp]
        L.synth_int_bytes.argtypes = [u64, u64, u64, i64, ctypes.c_int, ctypes.c_int, vp]
        L.synth_categorical.argtypes = [u64, u64, u64, i64, ctypes.c_uint32, vp]
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_expert_blob.argtypes = [u64, u64, u64, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_bf16(seed: int, stream: int, std: float, shape, first: int = 0, out=None) -> np.ndarray:
    """bf16 bit patterns (uint16) of std * N(0,1), element j from draw pair (first+j)."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16(seed, stream, std, first, n, _ptr(out))
    return out


def expert_record_bytes(d_latent: int, d_ffn: int) -> int:
    """Bytes of one expert record: 3 matrices of d_latent*d_ffn weights at 4 bits
    plus one byte per 32 weights."""
    return 3 * (d_latent * d_ffn // 2 + d_latent * d_ffn // 32)


def expert_blob(seed: int, d_latent: int, d_ffn: int, num_experts: int, out=None,
                scale_lo: int = SCALE_LO, scale_hi: int = SCALE_HI) -> np.ndarray:
    rec = expert_record_bytes(d_latent, d_ffn)
    if out is None:
        out = np.empty(num_experts * rec, dtype=np.uint8)
    assert out.nbytes == num_experts * rec
    lib().synth_expert_blob(seed, S_CODES, S_SCALES, d_latent, d_ffn, 0, num_experts,
                            scale_lo, scale_hi, _ptr(out))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, stream, n, _ptr(out))
    return out


def categorical(seed: int, stream: int, n: int, m: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_categorical(seed, stream, 0, n, m, _ptr(out))
    return out


@dataclass(frozen=True)
class Config:
    name: str
    T: int          # tokens
    d: int          # d_model (residual width)
    L: int          # latent width
    F: int          # expert ffn width
    E: int          # routed experts
    k: int          # experts per token
    layer_seed: int  # seeds the layer's weights (router, latent projections, expert blob)
    seed: int        # seeds the tokens and the router bias
    bias: Optional[str]  # None, "zipf" ([E] broadcast) or "domains" ([T, E])
    description: str

    @property
    def record_bytes(self) -> int:
        return expert_record_bytes(self.L, self.F)

    @property
    def blob_bytes(self) -> int:
        return self.E * self.record_bytes


_K3 = dict(d=7168, L=3584, F=3072, E=896, k=16, layer_seed=0x4B331000)

CONFIGS = {
    "tiny": Config("tiny", 16, 256, 128, 128, 8, 2, 0x4B330000, 0x4B330000, None,
                   "Tiny MoE layer: 16 tokens, d_model=256, latent=128, 8 experts top-2, expert ffn=128"),
    "decode1": Config("decode1", 1, seed=0x4B330001, bias=None,
                      description="K3-shape decode, 1 token: d_model=7168, latent=3584, 896 experts top-16, ffn=3072",
                      **_K3),
    "decode64": Config("decode64", 64, seed=0x4B330002, bias=None,
                       description="K3-shape decode batch of 64 tokens, same layer", **_K3),
    "prefill4k": Config("prefill4k", 4096, seed=0x4B330003, bias="zipf",
                        description="K3-shape prefill of 4096 tokens, per-expert router bias -1.1*ln(rank) (Zipf s=1.1)",
                        **_K3),
    "prefill32k": Config("prefill32k", 32768, seed=0x4B330004, bias="domains",
                         description="K3-shape prefill of 32768 tokens, 4 token domains each favouring its own "
                                     "224-expert cluster by +2.0 logit bias", **_K3),
}


def make_bias(cfg: Config, T: Optional[int] = None):
    """Router bias for a config: None, fp32 [E] (Zipf over a seeded expert ranking),
    or fp32 [T, E] (+2.0 on the experts of the token's domain cluster)."""
    T = cfg.T if T is None else T
    if cfg.bias is None:
        return None
    if cfg.bias == "zipf":
        rank = permutation(cfg.seed, S_ZIPF, cfg.E).astype(np.float64) + 1.0
        return (-1.1 * np.log(rank)).astype(np.float32)
    if cfg.bias == "domains":
        n_dom = 4
        dom = categorical(cfg.seed, S_DOMAIN, T, n_dom)
        perm = permutation(cfg.seed, S_CLUSTER, cfg.E)
        cluster = np.empty(cfg.E, dtype=np.int32)
        cluster[perm] = np.arange(cfg.E, dtype=np.int32) // (cfg.E // n_dom)
        return np.where(cluster[None, :] == dom[:, None], np.float32(2.0), np.float32(0.0)).astype(np.float32)
    raise ValueError(cfg.bias)


def make_tokens(cfg: Config, T: Optional[int] = None, first_token: int = 0, out=None) -> np.ndarray:
    """x: bf16 bits [T, d] ~ N(0, 1); token t is draw block (first_token + t)."""
    T = cfg.T if T is None else T
    return normal_bf16(cfg.seed, S_X, 1.0, (T, cfg.d), first=first_token * cfg.d, out=out)


def make_dense(cfg: Config) -> dict:
    """bf16 router [E, d], latent_down [L, d], latent_up [d, L], all ~ N(0, 0.02)."""
    s = cfg.layer_seed
    return dict(
        router_w=normal_bf16(s, S_ROUTER, 0.02, (cfg.E, cfg.d)),
        latent_down=normal_bf16(s, S_DOWN, 0.02, (cfg.L, cfg.d)),
        latent_up=normal_bf16(s, S_UP, 0.02, (cfg.d, cfg.L)),
    )


def make_blob(cfg: Config, out=None) -> np.ndarray:
    return expert_blob(cfg.layer_seed, cfg.L, cfg.F, cfg.E, out=out)


def make_layer(cfg: Config, blob_out=None) -> dict:
    """All inputs of a config as numpy arrays (bf16 as uint16 bit patterns)."""
    d = make_dense(cfg)
    d["x"] = make_tokens(cfg)
    d["bias"] = make_bias(cfg)
    d["blob"] = make_blob(cfg, out=blob_out)
    return d


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


__all__ = ["CONFIGS", "Config", "make_layer", "make_tokens", "make_dense", "make_blob", "make_bias",
           "normal_bf16", "expert_blob", "expert_record_bytes", "permutation", "categorical",
           "bf16_to_f32", "build", "lib"]
