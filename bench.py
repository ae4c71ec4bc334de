#!/usr/bin/env python3
"""Throughput of one Kimi-K3-shaped Stable-LatentMoE layer with MXFP4 experts on one MI355X.

One step = one pass of the whole layer (router, latent down projection, top-k,
permutation, MXFP4 gate/up with the fp32 GLU, MXFP4 down, combine, latent up)
over one batch of synthetic tokens, through the C ABI (moe_layer_forward).

The timed region replays one HIP graph per token batch, captured from the same C-ABI
call (--no-graph times the eager calls instead; both are reported): decode steps are
short enough that host launch overhead would otherwise show.

Inputs are resident in HBM before the timed region.  So that a step does not find
the previous step's weights in the 256 MB Infinity Cache, step i takes token
batch i (distinct tokens route to distinct experts) and dense-weight copy
i mod --dense-copies.

Prints one JSON line (rank 0).  The roofline object covers the dominant kernel
(the MXFP4 gate/up GEMV for decode): algorithmic bytes per launch over its mean
duration, measured with HIP events recorded around it on the layer's stream
inside the timed region.  cpu_baseline times the C oracle on the host.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X; HBM GB/s (decode), FP4 MFMA util (prefill)"
HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFS = 10100.0  # dense MFMA, fp4
FP8_PEAK_TFS = 5000.0   # dense MFMA, fp8
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEventCreate / hipEventElapsedTime through the HIP runtime."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


def recorded_traffic(config: str, packed: bool):
    """HBM bytes per gate/up launch from the counter summary in profiles/, if it was taken
    on this workload from the current sources of the expert kernels (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{config}_hbm_counters.md")
    if not packed or not os.path.exists(path):
        return None
    csrc = os.path.join(ROOT, "mxfp4_expert_gemm_amd", "csrc")
    names = ("expert_mfma.hip", "mfma_stream.h", "common.h", "kernels.h")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in names)
    fields = dict(line.split(": ", 1) for line in open(path).read().splitlines() if ": " in line)
    if fields.get(f"source_sha256 ({' + '.join(names)})") != hashlib.sha256(src).hexdigest():
        return None
    return int(fields["gate_up_traffic_bytes"])


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode1", choices=["decode1", "decode64", "prefill4k", "prefill32k", "tiny"])
    ap.add_argument("--dense-copies", type=int, default=3)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0, help="0 skips the oracle baseline")
    ap.add_argument("--breakdown", action="store_true", help="also time every stage (extra untimed pass)")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="time replays of HIP graphs captured from the layer call, one per token batch "
                         "(default); --no-graph times the eager calls")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes 5 times (calibrates HBM byte counters)")
    ap.add_argument("--act-format", default="bf16", choices=["bf16", "mxfp8"],
                    help="expert GEMM inputs: the bf16 activations (default) or their MXFP8 quantisation")
    ap.add_argument("--shared", type=int, default=0,
                    help="always-on shared experts of FFN width d_ffn (the routed layer alone by default)")
    ap.add_argument("--layout", default="packed", choices=["packed", "record"],
                    help="expert weights as packed once by moe_pack_experts (default) or as checkpoint records")
    ap.add_argument("--experts-in", default="hbm", choices=["hbm", "host"],
                    help="expert records resident in HBM (default) or in pinned host memory, the routed ones "
                         "fetched over the host link every step (moe_layer_forward_streamed)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs the layer on one GPU only: this build has no multi-GPU path "
              "(expert-parallel sharding is a design note, not code). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 5}), flush=True)
        return

    import mxfp4_expert_gemm_amd as moe
    import synth

    c = synth.CONFIGS[args.config]
    K, W = args.steps, args.warmup
    nbatch = K + W
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    t0 = time.time()
    dense = synth.make_dense(c)
    log(f"[bench] config {c.name}: T={c.T} d={c.d} L={c.L} F={c.F} E={c.E} k={c.k}; generating inputs")
    blob_host = synth.make_blob(c)
    blob = up(blob_host)
    packed = args.layout == "packed"
    if packed:  # a one-time reordering at load, outside the timed region
        blob = moe.pack_experts(blob, c.E, c.L, c.F)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    streamed = args.experts_in == "host"
    if streamed:  # the experts move to pinned host memory; HBM keeps only the slots
        if args.shared:
            raise SystemExit("--experts-in host runs the routed layer only (no --shared)")
        host_blob = torch.empty(blob.numel(), dtype=torch.uint8, pin_memory=True)
        host_blob.copy_(blob)
        del blob
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        blob = host_blob
    copies = [dict(router_w=up(dense["router_w"]), latent_down=up(dense["latent_down"]),
                   latent_up=up(dense["latent_up"])) for _ in range(max(1, args.dense_copies))]
    x_host = synth.make_tokens(c, T=c.T * nbatch).reshape(nbatch, c.T, c.d)
    xs = up(x_host)
    bias_host = synth.make_bias(c)
    bias = None if bias_host is None else up(bias_host)
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f}s)")

    act_format = moe.ACT_FMT_MXFP8 if args.act_format == "mxfp8" else moe.ACT_FMT_BF16
    shared = None
    if args.shared > 0:
        shared = up(synth.expert_blob(c.layer_seed + 77, c.d, c.F, args.shared))
        if packed:
            shared = moe.pack_experts(shared, args.shared, c.d, c.F)
    cfg = moe.make_config(c.T, c.d, c.L, c.F, c.E, bias=bias, packed=packed, act_format=act_format,
                          num_shared=args.shared, d_ffn_shared=c.F if args.shared else 0)
    ws = moe.alloc_workspace(cfg, c.k, dev)
    slots = moe.alloc_expert_slots(cfg, c.k, dev) if streamed else None
    out = torch.empty((c.T, c.d), dtype=torch.int16, device=dev)
    counts = torch.zeros((nbatch, c.E), dtype=torch.int32, device=dev)
    hip = HipEvents()
    ev_start, ev_stop = hip.create(2)
    dom = moe.STAGES.index("gate_up")
    kev = hip.create(2 * nbatch)

    def step(i, events=None):
        cp = copies[i % len(copies)]
        routing = {"expert_counts": counts[i]}
        if streamed:
            moe.layer_forward_streamed(xs[i], cp["router_w"], cp["latent_down"], cp["latent_up"], blob, c.k,
                                       d_ffn=c.F, expert_slots=slots, bias=bias, out=out, workspace=ws,
                                       routing=routing, packed=packed, act_format=act_format)
        elif events is None or args.shared:  # the stage events are not recorded with shared experts
            moe.layer_forward(xs[i], cp["router_w"], cp["latent_down"], cp["latent_up"], blob, c.k, d_ffn=c.F,
                              bias=bias, out=out, workspace=ws, routing=routing, packed=packed,
                              act_format=act_format, shared_blob=shared, num_shared=args.shared,
                              d_ffn_shared=c.F if args.shared else 0)
        else:
            moe.layer_forward_profiled(xs[i], cp["router_w"], cp["latent_down"], cp["latent_up"], blob, c.k,
                                       events, d_ffn=c.F, bias=bias, out=out, workspace=ws, routing=routing,
                                       packed=packed, act_format=act_format)

    def dom_events(i):
        ev = moe.StageEvents()
        ev.begin[dom] = kev[2 * i]
        ev.end[dom] = kev[2 * i + 1]
        return ev

    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # eager pass: warm-up, then K timed calls with events around the dominant kernel
    for i in range(W):
        step(i, dom_events(i))
    torch.cuda.synchronize()
    hip.rt.hipEventRecord(ev_start, stream)
    for i in range(W, W + K):
        step(i, dom_events(i))
    hip.rt.hipEventRecord(ev_stop, stream)
    torch.cuda.synchronize()
    eager_ms = hip.elapsed_ms(ev_start, ev_stop)
    dom_ms = ([hip.elapsed_ms(kev[2 * i], kev[2 * i + 1]) for i in range(W, W + K)]
              if not (args.shared or streamed) else [float("nan")] * K)

    total_ms = eager_ms
    if args.graph:
        # the warm-up batches and the K timed batches each captured into one graph, as a
        # model graph would run the layer (the library launches on the capturing stream and
        # neither allocates nor synchronises); every step still processes its own batch
        graphs = []
        for lo, hi in ((0, W), (W, W + K)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(lo, hi):
                    step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        graphs[0].replay()
        torch.cuda.synchronize()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        hip.rt.hipEventRecord(ev_start, stream)
        graphs[1].replay()
        hip.rt.hipEventRecord(ev_stop, stream)
        torch.cuda.synchronize()
        total_ms = hip.elapsed_ms(ev_start, ev_stop)
        del graphs
    ms_per_step = total_ms / K

    # algorithmic bytes of the dominant kernel per launch: gate and up codes+scales of every
    # active expert, the latent rows it reads and the GLU rows it writes
    cnt = counts.cpu().numpy()[W:W + K]
    # bytes of one gate (or up) matrix in the layout streamed (the same for the K3 shapes)
    mat_bytes = (moe.packed_expert_bytes(c.L, c.F) if packed else moe.expert_bytes(c.L, c.F)) // 3
    active = (cnt > 0).sum(1)
    dom_bytes = active * 2 * mat_bytes + c.T * c.L * 2 + c.T * c.k * c.F * 2
    dom_gbs = float(np.mean(dom_bytes / (np.array(dom_ms) * 1e-3)) / 1e9)
    # whole-layer algorithmic bytes: weights read (dense + active experts) + x + out + bias
    dense_bytes = (c.E * c.d + 2 * c.L * c.d) * 2
    layer_bytes = dense_bytes + active * 3 * mat_bytes + 2 * c.T * c.d * 2
    if bias_host is not None:
        layer_bytes = layer_bytes + bias_host.nbytes
    layer_gbs = float(np.mean(layer_bytes) / (ms_per_step * 1e-3) / 1e9)

    stages = None
    if args.breakdown and not (args.shared or streamed):
        evs = hip.create(2 * moe.NUM_STAGES)
        sums = np.zeros(moe.NUM_STAGES)
        n = min(K, 10)
        for i in range(W, W + n):
            ev = moe.StageEvents()
            for s in range(moe.NUM_STAGES):
                ev.begin[s] = evs[2 * s]
                ev.end[s] = evs[2 * s + 1]
            step(i, ev)
            torch.cuda.synchronize()
            sums += [hip.elapsed_ms(evs[2 * s], evs[2 * s + 1]) for s in range(moe.NUM_STAGES)]
        stages = {name: round(1e3 * v / n, 2) for name, v in zip(moe.STAGES, sums)}
        hip.destroy(evs)

    cpu = None
    if args.cpu_baseline_seconds > 0:
        import oracle

        budget = args.cpu_baseline_seconds
        t1 = time.time()
        n = 0
        xb = np.ascontiguousarray(x_host.reshape(nbatch * c.T, c.d)[: c.T])  # the first batch
        while True:
            oracle.layer_forward(xb, dense["router_w"], dense["latent_down"], dense["latent_up"], blob_host, c.k, c.L,
                                 c.F, bias=bias_host, tokens=[n % c.T])
            n += 1
            if time.time() - t1 >= budget:
                break
        dt = time.time() - t1
        cpu = {"value": round(n / dt, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} tokens of the {c.name} workload, whole layer one token at a time "
                         f"(single-threaded C oracle, fp64 sums, exact router), {dt:.1f} s"}

    if streamed:
        # the step is bound by the host link: the routed records cross it every step
        link_bytes = active * 3 * mat_bytes
        link_gbs = float(np.mean(link_bytes) / (ms_per_step * 1e-3) / 1e9)
        roofline = {"bound": "host link", "kernel": "gather_experts_kernel (routed records, pinned host -> HBM)",
                    "achieved": round(link_gbs, 1), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                    "frac": round(link_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                    "note": "achieved = routed record bytes per step / whole step time (a lower bound on the link rate)",
                    "bytes_per_step": int(np.mean(link_bytes))}
    elif c.T * c.k >= 8 * c.E:
        # many routed rows per expert: the gate/up stage runs as grouped GEMMs on the matrix
        # cores; model flops 2 x rows x F x L per matrix against the dense FP4 peak (the
        # kernel issues e4m3 x e2m1 MFMAs, two per K step, at the fp8 rate)
        flops = 2 * 2 * c.T * c.k * c.F * c.L
        tfs = flops / (float(np.mean(dom_ms)) * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "gate_up (grouped MXFP4 GEMM + fp32 GLU)", "achieved": round(tfs, 1),
                    "peak": FP4_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / FP4_PEAK_TFS, 4), "traffic": None,
                    "kernel_us": round(1e3 * float(np.mean(dom_ms)), 2), "flops_per_launch": flops,
                    "issued_vs_fp8_peak": round((2 if args.act_format == "bf16" else 1) * tfs / FP8_PEAK_TFS, 4)}
    else:
        roofline = {"bound": "hbm", "kernel": "gate_up (MXFP4 gate/up GEMV + fp32 GLU)",
                    "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(c.name, packed),
                    "kernel_us": round(1e3 * float(np.mean(dom_ms)), 2), "bytes_per_launch": int(np.mean(dom_bytes))}

    tokens_per_s = c.T * K / (total_ms * 1e-3)
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "timing": ("one replay of a HIP graph holding the K steps (each on its own token batch)" if args.graph
                   else "eager calls"),
        "eager_ms_per_step": round(eager_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.act_format == "bf16" else "bf16 dense, mxfp8 x mxfp4 experts",
        "data": "synthetic",
        "config": {"workload": f"{c.name}: {c.description}", "tokens": c.T, "d_model": c.d, "d_latent": c.L,
                   "d_ffn": c.F, "experts": c.E, "top_k": c.k, "expert_weights": "mxfp4 (e2m1 + e8m0 per 32)",
                   "activations": ("bf16, fp32 accumulation, fp32 GLU" if args.act_format == "bf16" else
                                   "MXFP8 (e4m3 + e8m0 per 32) at the expert GEMM inputs, fp32 accumulation, fp32 GLU"),
                   "parallelism": "single GPU",
                   "dense_weight_copies": len(copies), "mean_active_experts": float(np.mean(active)),
                   "shared_experts": args.shared,
                   "expert_layout": "packed by moe_pack_experts at load" if packed else "checkpoint records",
                   "experts_in": "pinned host memory, routed records fetched per step" if streamed else "HBM"},
        "roofline": roofline,
        "layer_hbm": {"achieved_GBs": round(layer_gbs, 1), "frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_step": int(np.mean(layer_bytes))},
        "cpu_baseline": cpu,
    }
    if stages is not None:
        result["stages_us"] = stages
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
