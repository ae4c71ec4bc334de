"""Python binding of libmoe_layer.so: the MI355X (gfx950) MXFP4 Stable-LatentMoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  bf16 tensors
may be torch.bfloat16 or int16/uint16 tensors holding bf16 bit patterns.

The library is built in-tree by ``python -m mxfp4_expert_gemm_amd.build``; if
it is missing, importing this package's functions raises instead of falling
back to any other implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_layer.so")

ACT_SILU, ACT_SITU = 0, 1
ROUTE_EXACT_ALL = 1
LAYOUT_RECORD, LAYOUT_PACKED = 0, 1
ACT_FMT_BF16, ACT_FMT_MXFP8 = 0, 1  # activation format at the expert GEMM inputs
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE",
          -4: "MOE_ERR_DEVICE"}
EXPORTS = ["moe_expert_bytes", "moe_packed_expert_bytes", "moe_pack_experts", "moe_status_string",
           "moe_workspace_size", "moe_layer_forward",
           "moe_layer_forward_profiled",
           "moe_dequant_mxfp4", "moe_route", "moe_topk", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_linear_bf16", "moe_reap_saliency", "moe_layer_forward_shared", "moe_expert_slots_bytes",
           "moe_layer_forward_streamed", "moe_layer_forward_noalloc", "moe_reap_keep_bias",
           "moe_permute_workspace_size"]


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class MoEConfig(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_ffn", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("act", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("bias_row_stride", ctypes.c_int64),
                ("expert_layout", ctypes.c_int32), ("act_format", ctypes.c_int32), ("num_shared", ctypes.c_int32),
                ("d_ffn_shared", ctypes.c_int32)]


NUM_STAGES = 7
CLOCK_SLOTS = 1024  # MOE_CLOCK_SLOTS: {start, end} uint64 pairs behind each kernel_clock pointer
STAGES = ["router_down", "route", "permute", "gate_up", "down", "combine", "up"]


class StageEvents(ctypes.Structure):
    """moe_stage_events: events recorded around each stage (begin/end), events the dispatch
    of a stage's main kernel stamps at its start and end (kernel_begin/kernel_end), and
    device pointers to CLOCK_SLOTS {start, end} uint64 pairs the main kernel's blocks stamp
    with the device wall clock (kernel_clock; gate/up and down stages)."""
    _fields_ = [("begin", ctypes.c_void_p * NUM_STAGES), ("end", ctypes.c_void_p * NUM_STAGES),
                ("kernel_begin", ctypes.c_void_p * NUM_STAGES), ("kernel_end", ctypes.c_void_p * NUM_STAGES),
                ("kernel_clock", ctypes.c_void_p * NUM_STAGES)]


class RoutingOut(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("saliency", ctypes.c_void_p)]


_lib = None


def lib():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_expert_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp, rp = ctypes.POINTER(MoEConfig), ctypes.POINTER(RoutingOut)
        sig = {
            "moe_expert_bytes": (sz, [i32, i32]),
            "moe_packed_expert_bytes": (sz, [i32, i32]),
            "moe_pack_experts": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_workspace_size": (ctypes.c_int, [cfgp, i32, ctypes.POINTER(sz)]),
            "moe_layer_forward": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, cfgp, vp, vp, rp, vp, sz, vp]),
            "moe_layer_forward_profiled": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, cfgp, vp, vp, rp, vp, sz,
                                                          ctypes.POINTER(StageEvents), vp]),
            "moe_dequant_mxfp4": (ctypes.c_int, [vp, vp, i64, i32, vp, vp]),
            "moe_route": (ctypes.c_int, [vp, vp, vp, cfgp, i32, i32, rp, vp, sz, vp]),
            "moe_topk": (ctypes.c_int, [vp, i64, i32, i32, i32, vp, vp, vp]),
            "moe_permute": (ctypes.c_int, [vp, i64, i32, i32, vp, vp, vp, vp, sz, vp]),
            "moe_permute_workspace_size": (ctypes.c_int, [i64, i32, i32, ctypes.POINTER(sz)]),
            "moe_expert_ffn": (ctypes.c_int, [vp, vp, i32, cfgp, rp, vp, vp, vp, sz, vp]),
            "moe_combine": (ctypes.c_int, [vp, vp, i64, i32, i32, vp, vp]),
            "moe_linear_bf16": (ctypes.c_int, [vp, vp, i64, i32, i32, vp, vp]),
            "moe_reap_saliency": (ctypes.c_int, [vp, vp, vp, vp, i64, i32, i32, i32, vp, vp]),
            "moe_reap_keep_bias": (ctypes.c_int, [vp, i32, i32, vp, vp]),
            "moe_layer_forward_shared": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, cfgp, vp, vp, vp, rp, vp, sz, vp]),
            "moe_expert_slots_bytes": (ctypes.c_int, [cfgp, i32, ctypes.POINTER(sz)]),
            "moe_layer_forward_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, cfgp, vp, vp, rp, vp]),
            "moe_layer_forward_streamed": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, cfgp, vp, vp, sz, vp, rp, vp, sz,
                                                          vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise MoEError(status, what)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_config(num_tokens: int, d_model: int, d_latent: int, d_ffn: int, num_experts: int, *,
                act: int = ACT_SILU, renormalize: bool = True, bias: Optional[torch.Tensor] = None,
                packed: bool = False, act_format: int = ACT_FMT_BF16, num_shared: int = 0,
                d_ffn_shared: int = 0) -> MoEConfig:
    stride = 0 if bias is None or bias.dim() == 1 else num_experts
    return MoEConfig(num_tokens, d_model, d_latent, d_ffn, num_experts, act, int(renormalize), stride,
                     LAYOUT_PACKED if packed else LAYOUT_RECORD, act_format, num_shared, d_ffn_shared)


def expert_bytes(d_latent: int, d_ffn: int) -> int:
    return int(lib().moe_expert_bytes(d_latent, d_ffn))


def packed_expert_bytes(d_latent: int, d_ffn: int) -> int:
    return int(lib().moe_packed_expert_bytes(d_latent, d_ffn))


def pack_experts(blob: torch.Tensor, num_experts: int, d_latent: int, d_ffn: int,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The experts of a checkpoint blob in the packed layout (see moe_pack_experts)."""
    if out is None:
        out = torch.empty(num_experts * packed_expert_bytes(d_latent, d_ffn), dtype=torch.uint8, device=blob.device)
    _check(lib().moe_pack_experts(_p(blob), num_experts, d_latent, d_ffn, _p(out), _stream()), "moe_pack_experts")
    return out


def workspace_size(cfg: MoEConfig, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), k, ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


def alloc_workspace(cfg: MoEConfig, k: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(cfg, k), 256), dtype=torch.uint8, device=device)


def _routing(r: Optional[dict]) -> Optional[RoutingOut]:
    if r is None:
        return None
    return RoutingOut(*[_p(r.get(n)) for n in ("topk_idx", "topk_w", "logits", "expert_counts", "expert_offsets",
                                              "perm", "saliency")])


def layer_forward(x, router_w, latent_down, latent_up, expert_blob, k: int, *, d_ffn: int,
                  bias: Optional[torch.Tensor] = None, renormalize: bool = True, act: int = ACT_SILU,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  routing: Optional[dict] = None, stream=None, packed: bool = False,
                  act_format: int = ACT_FMT_BF16, shared_blob: Optional[torch.Tensor] = None,
                  num_shared: int = 0, d_ffn_shared: int = 0) -> torch.Tensor:
    """out = layer(x); routing (dict of preallocated tensors) receives the routing if given;
    shared_blob with num_shared records of width d_ffn_shared adds the shared experts."""
    T, d = x.shape
    E = router_w.shape[0]
    L = latent_down.shape[0]
    cfg = make_config(T, d, L, d_ffn, E, act=act, renormalize=renormalize, bias=bias, packed=packed,
                      act_format=act_format, num_shared=num_shared, d_ffn_shared=d_ffn_shared)
    if out is None:
        out = torch.empty((T, d), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, k, x.device)
    r = _routing(routing)
    if num_shared > 0:
        _check(lib().moe_layer_forward_shared(_p(x), _p(router_w), _p(latent_down), _p(latent_up), _p(expert_blob),
                                              k, ctypes.byref(cfg), _p(bias), _p(shared_blob), _p(out),
                                              ctypes.byref(r) if r else None, _p(workspace), workspace.numel(),
                                              _stream(stream)), "moe_layer_forward_shared")
    else:
        _check(lib().moe_layer_forward(_p(x), _p(router_w), _p(latent_down), _p(latent_up), _p(expert_blob), k,
                                       ctypes.byref(cfg), _p(bias), _p(out), ctypes.byref(r) if r else None,
                                       _p(workspace), workspace.numel(), _stream(stream)), "moe_layer_forward")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def layer_forward_noalloc(x, router_w, latent_down, latent_up, expert_blob, k: int, *, d_ffn: int, out: torch.Tensor,
                          bias: Optional[torch.Tensor] = None, renormalize: bool = True, act: int = ACT_SILU,
                          routing: Optional[dict] = None, stream=None, packed: bool = False,
                          act_format: int = ACT_FMT_BF16) -> torch.Tensor:
    """layer_forward without a workspace (moe_layer_forward_noalloc): the library's own device
    scratch serves, and nothing is allocated here either, so `out` (and any routing tensors)
    must be given.  Calls that overlap on one GPU race on that scratch."""
    T, d = x.shape
    cfg = make_config(T, d, latent_down.shape[0], d_ffn, router_w.shape[0], act=act, renormalize=renormalize,
                      bias=bias, packed=packed, act_format=act_format)
    r = _routing(routing)
    _check(lib().moe_layer_forward_noalloc(_p(x), _p(router_w), _p(latent_down), _p(latent_up), _p(expert_blob), k,
                                           ctypes.byref(cfg), _p(bias), _p(out), ctypes.byref(r) if r else None,
                                           _stream(stream)), "moe_layer_forward_noalloc")
    return out


def expert_slots_bytes(cfg: MoEConfig, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_expert_slots_bytes(ctypes.byref(cfg), k, ctypes.byref(n)), "moe_expert_slots_bytes")
    return int(n.value)


def alloc_expert_slots(cfg: MoEConfig, k: int, device="cuda") -> torch.Tensor:
    """The HBM slot buffer of moe_layer_forward_streamed for this batch shape."""
    return torch.empty(max(expert_slots_bytes(cfg, k), 256), dtype=torch.uint8, device=device)


def layer_forward_streamed(x, router_w, latent_down, latent_up, expert_blob_host: torch.Tensor, k: int, *,
                           d_ffn: int, expert_slots: Optional[torch.Tensor] = None,
                           bias: Optional[torch.Tensor] = None, renormalize: bool = True, act: int = ACT_SILU,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           routing: Optional[dict] = None, stream=None, packed: bool = False,
                           act_format: int = ACT_FMT_BF16) -> torch.Tensor:
    """layer_forward with the expert records in pinned host memory (expert_blob_host, a CPU
    tensor with pin_memory): the routed experts are fetched into expert_slots (HBM) on the
    device before the expert kernels run."""
    if expert_blob_host.is_cuda or not expert_blob_host.is_pinned():
        raise ValueError("expert_blob_host must be a pinned host tensor")
    T, d = x.shape
    E = router_w.shape[0]
    L = latent_down.shape[0]
    cfg = make_config(T, d, L, d_ffn, E, act=act, renormalize=renormalize, bias=bias, packed=packed,
                      act_format=act_format)
    if out is None:
        out = torch.empty((T, d), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, k, x.device)
    if expert_slots is None:
        expert_slots = alloc_expert_slots(cfg, k, x.device)
    r = _routing(routing)
    _check(lib().moe_layer_forward_streamed(_p(x), _p(router_w), _p(latent_down), _p(latent_up),
                                            expert_blob_host.data_ptr(), k, ctypes.byref(cfg), _p(bias),
                                            _p(expert_slots), expert_slots.numel(), _p(out),
                                            ctypes.byref(r) if r else None, _p(workspace), workspace.numel(),
                                            _stream(stream)), "moe_layer_forward_streamed")
    return out


def layer_forward_profiled(x, router_w, latent_down, latent_up, expert_blob, k: int, events: "StageEvents", *,
                           d_ffn: int, bias: Optional[torch.Tensor] = None, renormalize: bool = True,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           routing: Optional[dict] = None, stream=None, packed: bool = False,
                           act_format: int = ACT_FMT_BF16) -> torch.Tensor:
    """layer_forward that records the caller's HIP events around each stage (see StageEvents)."""
    T, d = x.shape
    cfg = make_config(T, d, latent_down.shape[0], d_ffn, router_w.shape[0], renormalize=renormalize, bias=bias,
                      packed=packed, act_format=act_format)
    if out is None:
        out = torch.empty((T, d), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, k, x.device)
    r = _routing(routing)
    _check(lib().moe_layer_forward_profiled(_p(x), _p(router_w), _p(latent_down), _p(latent_up), _p(expert_blob), k,
                                            ctypes.byref(cfg), _p(bias), _p(out), ctypes.byref(r) if r else None,
                                            _p(workspace), workspace.numel(), ctypes.byref(events), _stream(stream)),
           "moe_layer_forward_profiled")
    return out


def dequant_mxfp4(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    _check(lib().moe_dequant_mxfp4(_p(codes), _p(scales), rows, cols, _p(out), _stream()), "moe_dequant_mxfp4")
    return out


def route(x, router_w, k: int, *, bias=None, renormalize: bool = True, flags: int = 0, workspace=None,
          d_latent: int = 128, d_ffn: int = 128):
    """Exact routing: returns (logits [T,E], idx [T,k], w [T,k])."""
    T, d = x.shape
    E = router_w.shape[0]
    cfg = make_config(T, d, d_latent, d_ffn, E, renormalize=renormalize, bias=bias)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, k, x.device)
    r = RoutingOut(idx.data_ptr(), w.data_ptr(), logits.data_ptr(), None, None, None)
    _check(lib().moe_route(_p(x), _p(router_w), _p(bias), ctypes.byref(cfg), k, flags, ctypes.byref(r),
                           _p(workspace), workspace.numel(), _stream()), "moe_route")
    return logits, idx, w


def topk(logits: torch.Tensor, k: int, renormalize: bool = True):
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_topk(_p(logits), T, E, k, int(renormalize), _p(idx), _p(w), _stream()), "moe_topk")
    return idx, w


def permute(idx: torch.Tensor, num_experts: int):
    T, k = idx.shape
    counts = torch.empty(num_experts, dtype=torch.int32, device=idx.device)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=idx.device)
    perm = torch.empty(T * k, dtype=torch.int32, device=idx.device)
    n = ctypes.c_size_t(0)
    _check(lib().moe_permute_workspace_size(T, k, num_experts, ctypes.byref(n)), "moe_permute_workspace_size")
    ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=idx.device)
    _check(lib().moe_permute(_p(idx), T, k, num_experts, _p(counts), _p(offsets), _p(perm), _p(ws), ws.numel(),
                             _stream()), "moe_permute")
    return counts, offsets, perm


def expert_ffn(h: torch.Tensor, expert_blob: torch.Tensor, idx: torch.Tensor, *, d_model: int, d_ffn: int,
               num_experts: int, want_a: bool = False, workspace=None, packed: bool = False,
               act_format: int = ACT_FMT_BF16, y: Optional[torch.Tensor] = None, a: Optional[torch.Tensor] = None):
    """Routed experts on latent rows h [T, L]: returns y fp32 [T*k, L] (and a bf16 [T*k, F]),
    into the given y and a when passed."""
    T, L = h.shape
    k = idx.shape[1]
    cfg = make_config(T, d_model, L, d_ffn, num_experts, packed=packed, act_format=act_format)
    if y is None:
        y = torch.empty((T * k, L), dtype=torch.float32, device=h.device)
    if a is None and want_a:
        a = torch.empty((T * k, d_ffn), dtype=h.dtype, device=h.device)
    want_a = a is not None
    if tuple(y.shape) != (T * k, L) or y.dtype != torch.float32 or not y.is_contiguous():
        raise ValueError(f"y must be a contiguous float32 [{T * k}, {L}] tensor")
    if want_a and (tuple(a.shape) != (T * k, d_ffn) or a.element_size() != 2 or not a.is_contiguous()):
        raise ValueError(f"a must be a contiguous 2-byte [{T * k}, {d_ffn}] tensor")
    if workspace is None:
        workspace = alloc_workspace(cfg, k, h.device)
    r = RoutingOut(idx.data_ptr(), None, None, None, None, None)
    _check(lib().moe_expert_ffn(_p(h), _p(expert_blob), k, ctypes.byref(cfg), ctypes.byref(r), _p(y), _p(a),
                                _p(workspace), workspace.numel(), _stream()), "moe_expert_ffn")
    return (y, a) if want_a else y


def combine(y: torch.Tensor, w: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    T, k = w.shape
    L = y.shape[1]
    z = torch.empty((T, L), dtype=dtype, device=y.device)
    _check(lib().moe_combine(_p(y), _p(w), T, k, L, _p(z), _stream()), "moe_combine")
    return z


def linear_bf16(inp: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
    T, n_in = inp.shape
    n_out = W.shape[0]
    out = torch.empty((T, n_out), dtype=inp.dtype, device=inp.device)
    _check(lib().moe_linear_bf16(_p(inp), _p(W), T, n_in, n_out, _p(out), _stream()), "moe_linear_bf16")
    return out


def reap_saliency(y: torch.Tensor, topk_w: torch.Tensor, perm: torch.Tensor, expert_offsets: torch.Tensor,
                  num_experts: int, saliency: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Adds the REAP score sums of these routed rows to saliency (fp64 [E], zeros if None)."""
    T, k = topk_w.shape
    if saliency is None:
        saliency = torch.zeros(num_experts, dtype=torch.float64, device=y.device)
    _check(lib().moe_reap_saliency(_p(y), _p(topk_w), _p(perm), _p(expert_offsets), T, k, y.shape[1], num_experts,
                                   _p(saliency), _stream()), "moe_reap_saliency")
    return saliency


def reap_prune_bias(saliency: torch.Tensor, n_keep: int) -> torch.Tensor:
    """Router bias of a REAP-pruned layer (moe_reap_keep_bias): 0 on the n_keep experts of
    highest saliency (ties to the lower index, NaN last), -inf on the others."""
    if saliency.dtype != torch.float64 or not saliency.is_contiguous():
        raise ValueError("saliency must be a contiguous fp64 tensor")
    E = saliency.numel()
    bias = torch.empty((E,), dtype=torch.float32, device=saliency.device)
    _check(lib().moe_reap_keep_bias(_p(saliency), E, n_keep, _p(bias), _stream()), "moe_reap_keep_bias")
    return bias


__all__ = ["lib", "MoEConfig", "RoutingOut", "MoEError", "make_config", "expert_bytes", "packed_expert_bytes",
           "pack_experts", "LAYOUT_RECORD", "LAYOUT_PACKED", "ACT_FMT_BF16", "ACT_FMT_MXFP8", "workspace_size",
           "alloc_workspace", "layer_forward", "layer_forward_profiled", "StageEvents", "STAGES", "dequant_mxfp4", "route", "topk", "permute", "expert_ffn", "combine",
           "linear_bf16", "reap_saliency", "reap_prune_bias", "ACT_SILU", "ACT_SITU", "ROUTE_EXACT_ALL", "EXPORTS",
           "LIB_PATH", "expert_slots_bytes", "alloc_expert_slots", "layer_forward_streamed", "layer_forward_noalloc",
           "NOALLOC_SCRATCH_BYTES"]
