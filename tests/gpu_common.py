"""Shared fixtures for the GPU parity tests: seeded layers on host (for the oracle)
and on the device (for the HIP library), built once per session."""
import functools
import os
import sys

import numpy as np
import torch

import synth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


@functools.lru_cache(maxsize=None)
def host_layer(name: str, T: int = None):
    """numpy inputs of a workload (bf16 as uint16); the K3 layers share one blob."""
    c = synth.CONFIGS[name]
    if c.d == 7168:
        dense = k3_dense()
        blob = k3_blob()
    else:
        dense = synth.make_dense(c)
        blob = synth.make_blob(c)
    x = synth.make_tokens(c, T=T)
    bias = synth.make_bias(c, T=T)
    return dict(cfg=c, x=x, bias=bias, blob=blob, **dense)


@functools.lru_cache(maxsize=None)
def k3_dense():
    return synth.make_dense(synth.CONFIGS["decode1"])


@functools.lru_cache(maxsize=None)
def k3_blob():
    log("generating the 15.7 GB K3 expert blob ...")
    return synth.make_blob(synth.CONFIGS["decode1"])


@functools.lru_cache(maxsize=None)
def dev_weights(name: str):
    h = host_layer(name)
    if h["cfg"].d == 7168:
        return k3_dev_weights()
    return dict(router_w=to_dev(h["router_w"]), latent_down=to_dev(h["latent_down"]),
                latent_up=to_dev(h["latent_up"]), blob=to_dev(h["blob"]))


@functools.lru_cache(maxsize=None)
def k3_dev_weights():
    d = k3_dense()
    log("uploading the K3 layer to the GPU ...")
    return dict(router_w=to_dev(d["router_w"]), latent_down=to_dev(d["latent_down"]),
                latent_up=to_dev(d["latent_up"]), blob=to_dev(k3_blob()))


@functools.lru_cache(maxsize=None)
def dev_packed(name: str):
    """The device blob of a workload in the packed expert layout."""
    import mxfp4_expert_gemm_amd as moe
    c = synth.CONFIGS[name]
    if c.d == 7168:
        name = "decode1"  # the K3 workloads share one blob
    t = moe.pack_experts(dev_weights(name)["blob"], c.E, c.L, c.F)
    torch.cuda.synchronize()
    return t


# worker threads for the oracle's token shards: the host share of one GPU is 16 cores
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@functools.lru_cache(maxsize=None)
def oracle_routing(name: str):
    """The oracle's routing of every token of a workload: (logits, idx, w), computed once
    per session on token shards side by side."""
    import oracle
    h = host_layer(name)
    c = h["cfg"]
    log(f"oracle routing of all {h['x'].shape[0]} {name} tokens on {ORACLE_THREADS} threads ...")
    logits = oracle.router_logits(h["x"], h["router_w"], h["bias"], threads=ORACLE_THREADS)
    idx, w = oracle.select(logits, c.k, threads=ORACLE_THREADS)
    return logits, idx, w
