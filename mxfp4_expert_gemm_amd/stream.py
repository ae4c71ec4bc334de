"""Layers whose experts do not all fit in HBM: prefix pinning and per-call streaming.

A Kimi K3 has 92 routed layers with 896 experts of 17,547,264 bytes each: 15.7 GB of
experts per layer and 1.45 TB in all (in-c post, section on how the memory requirement
shrinks), five times the 288 GB of one MI355X.  Two facts of that post decide the design:

* Only the experts a token routes to are needed: 16 of 896 per layer and token.  A layer
  whose records stay in pinned host memory runs through `layer_forward_streamed`, which
  copies just the routed records into HBM slots on the device before its expert kernels.
* Layers are visited in the same order for every token, a cyclic scan.  For that pattern
  a least-recently-used cache with fewer slots than layers never hits (the post's example:
  93 layers, 90 slots, hit rate 0), while pinning the first N layers guarantees N of every
  pass (90/93 = 96.8%).  So the first N layers keep their experts in HBM for good and the
  others stream (section on streaming the trunk, which applies it to the dense weights).

`plan_prefix` sizes N for an HBM budget, `cache_hits` replays the scan for either policy,
and `LayerStack` runs a stack with the first N layers resident and the rest streamed.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import List, Optional, Sequence

import torch

from . import alloc_expert_slots, alloc_workspace, layer_forward, layer_forward_streamed, make_config


def plan_prefix(num_layers: int, layer_expert_bytes: int, hbm_budget_bytes: int, reserved_bytes: int = 0) -> int:
    """Layers whose experts fit in the HBM budget after the reserved bytes (dense weights,
    workspace, slot buffer): the first N are pinned, N = min(num_layers, free // per layer)."""
    if num_layers < 0 or layer_expert_bytes <= 0:
        raise ValueError("num_layers >= 0 and layer_expert_bytes > 0")
    free = hbm_budget_bytes - reserved_bytes
    return max(0, min(num_layers, free // layer_expert_bytes))


def cache_hits(num_layers: int, passes: int, slots: int, policy: str) -> int:
    """Hits over `passes` scans of layers 0..num_layers-1 with `slots` layer-sized slots.
    policy 'lru': least recently used eviction; 'prefix': layers < slots pinned, the rest
    always fetched."""
    if policy == "prefix":
        return passes * min(slots, num_layers)
    if policy != "lru":
        raise ValueError(policy)
    cache: "OrderedDict[int, None]" = OrderedDict()
    hits = 0
    for _ in range(passes):
        for layer in range(num_layers):
            if layer in cache:
                hits += 1
                cache.move_to_end(layer)
                continue
            if slots == 0:
                continue
            if len(cache) >= slots:
                cache.popitem(last=False)
            cache[layer] = None
    return hits


class LayerStack:
    """A stack of MoE layers: dense weights in HBM, experts in HBM for the first `pinned`
    layers and in pinned host memory for the others.

    layers: per layer a dict with router_w, latent_down, latent_up (device bf16 tensors)
    and expert_blob_host (pinned host uint8 tensor, E records).  Layers may share tensors
    (the same object is uploaded once).  Every layer call uses one workspace and one slot
    buffer, sized for `num_tokens` tokens.
    """

    def __init__(self, layers: Sequence[dict], k: int, d_ffn: int, pinned: int, num_tokens: int, *,
                 packed: bool = False, device="cuda"):
        if not 0 <= pinned <= len(layers):
            raise ValueError("pinned must be in [0, number of layers]")
        self.layers = list(layers)
        self.k, self.d_ffn, self.pinned, self.packed = k, d_ffn, pinned, packed
        self.resident: List[Optional[torch.Tensor]] = []
        uploaded = {}
        for i, lay in enumerate(self.layers):
            host = lay["expert_blob_host"]
            if host.is_cuda or not host.is_pinned():
                raise ValueError(f"layer {i}: expert_blob_host must be a pinned host tensor")
            if i < pinned:
                key = host.data_ptr()
                if key not in uploaded:
                    uploaded[key] = host.to(device, non_blocking=False)
                self.resident.append(uploaded[key])
            else:
                self.resident.append(None)
        first = self.layers[0]
        T, d = num_tokens, first["router_w"].shape[1]
        cfg = make_config(T, d, first["latent_down"].shape[0], d_ffn, first["router_w"].shape[0], packed=packed)
        self.workspace = alloc_workspace(cfg, k, device)
        self.slots = alloc_expert_slots(cfg, k, device) if pinned < len(self.layers) else None
        self.num_tokens = T

    def forward_layer(self, i: int, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                      routing: Optional[dict] = None, stream=None) -> torch.Tensor:
        lay = self.layers[i]
        args = (x, lay["router_w"], lay["latent_down"], lay["latent_up"])
        kw = dict(d_ffn=self.d_ffn, bias=lay.get("bias"), out=out, workspace=self.workspace, routing=routing,
                  stream=stream, packed=self.packed)
        if self.resident[i] is not None:
            return layer_forward(*args, self.resident[i], self.k, **kw)
        return layer_forward_streamed(*args, lay["expert_blob_host"], self.k, expert_slots=self.slots, **kw)

    def step(self, xs: Sequence[torch.Tensor], outs: Optional[Sequence[torch.Tensor]] = None,
             stream=None) -> List[torch.Tensor]:
        """One pass over the stack: layer i on xs[i] (the hidden state each layer receives;
        attention and the residual stream between layers are not part of this path)."""
        if len(xs) != len(self.layers):
            raise ValueError("one input per layer")
        res = []
        for i, x in enumerate(xs):
            res.append(self.forward_layer(i, x, None if outs is None else outs[i], stream=stream))
        return res


__all__ = ["plan_prefix", "cache_hits", "LayerStack"]
