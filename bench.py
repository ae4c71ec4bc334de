#!/usr/bin/env python3
"""Throughput of one Kimi-K3-shaped Stable-LatentMoE layer with MXFP4 experts on one MI355X.

One step = one pass of the whole layer (router, latent down projection, top-k,
permutation, MXFP4 gate/up with the fp32 GLU, MXFP4 down, combine, latent up)
over one batch of synthetic tokens, through the C ABI (moe_layer_forward).

The headline is single-token decode (the HBM-bound half of the metric).  The default
run also measures the 4096-token prefill on the same synthesised layer (the
matrix-core half of the metric) and reports it in the same JSON line.

The timed region replays one HIP graph holding the K steps, captured from the same
C-ABI call (--no-graph times the eager calls instead; both are reported): decode
steps are short enough that host launch overhead would otherwise show.  Inputs are
resident in HBM before the timed region.  So that a step does not find the previous
step's weights in the 256 MB Infinity Cache, step i takes token batch i (distinct
tokens route to distinct experts) and dense-weight copy i mod --dense-copies; a
warm-cache figure (every step on one batch and one copy) is reported beside it.

The roofline object covers the dominant kernel (the MXFP4 gate/up kernel):
algorithmic bytes (decode) or model flops (prefill) per launch over its mean
duration.  The duration is the span the kernel stamps on the device's constant-rate
wall clock (earliest block start to latest wave end) in a second graph of the same K
steps, where the kernels run as in the timed graph; the eager pass's dispatch-stamped
events (hipExtLaunchKernelGGL) are reported beside it.  cpu_baseline times the C
oracle on the host.
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X; HBM GB/s (decode), FP4 MFMA util (prefill)"
HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFS = 10100.0   # dense MFMA, fp4
FP8_PEAK_TFS = 5000.0    # dense MFMA, fp8
BF16_PEAK_TFS = 2500.0   # dense MFMA, bf16
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction
HIP_ATTR_WALL_CLOCK_RATE = 10017  # hipDeviceAttributeWallClockRate in hip_runtime_api.h (kHz)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEventCreate / hipEventElapsedTime / hipEventRecord through the HIP runtime."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def record(self, e, stream):
        if self.rt.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)

    def wall_clock_khz(self, device=0):
        """Rate of the device's constant-rate wall clock (hipDeviceAttributeWallClockRate)."""
        v = ctypes.c_int(0)
        self.rt.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
        if self.rt.hipDeviceGetAttribute(ctypes.byref(v), HIP_ATTR_WALL_CLOCK_RATE, device) != 0 or v.value <= 0:
            raise RuntimeError("hipDeviceGetAttribute(hipDeviceAttributeWallClockRate) failed")
        return float(v.value)


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


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


class Layer:
    """The layer's weights on the device (one synthesised layer serves every K3 workload)."""

    def __init__(self, c, args, torch, moe, synth, dev):
        self.up = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        t0 = time.time()
        self.dense = synth.make_dense(c)
        log(f"[bench] layer d={c.d} L={c.L} F={c.F} E={c.E}: generating weights")
        self.blob_host = synth.make_blob(c)
        blob = self.up(self.blob_host)
        self.packed = args.layout == "packed"
        if self.packed:  # a one-time reordering at load, outside the timed region
            blob = moe.pack_experts(blob, c.E, c.L, c.F)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        self.streamed = args.experts_in == "host"
        if self.streamed:  # the experts move to pinned host memory; HBM keeps only the slots
            host_blob = torch.empty(blob.numel(), dtype=torch.uint8, pin_memory=True)
            host_blob.copy_(blob)
            del blob
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            blob = host_blob
        self.blob = blob
        self.copies = [dict(router_w=self.up(self.dense["router_w"]), latent_down=self.up(self.dense["latent_down"]),
                            latent_up=self.up(self.dense["latent_up"])) for _ in range(max(1, args.dense_copies))]
        self.shared = None
        if args.shared > 0:
            self.shared = self.up(synth.expert_blob(c.layer_seed + 77, c.d, c.F, args.shared))
            if self.packed:
                self.shared = moe.pack_experts(self.shared, args.shared, c.d, c.F)
        log(f"[bench] weights resident in HBM ({time.time() - t0:.1f}s)")


def run_config(c, layer, args, K, W, torch, moe, synth, dev, hip, warm=False):
    """Times K steps of the layer on workload c (after W warm-up steps); returns a dict."""
    nbatch = K + W
    act_format = moe.ACT_FMT_MXFP8 if args.act_format == "mxfp8" else moe.ACT_FMT_BF16
    x_host = synth.make_tokens(c, T=c.T * nbatch).reshape(nbatch, c.T, c.d)
    xs = layer.up(x_host)
    bias_host = synth.make_bias(c)
    bias = None if bias_host is None else layer.up(bias_host)
    cfg = moe.make_config(c.T, c.d, c.L, c.F, c.E, bias=bias, packed=layer.packed, act_format=act_format,
                          num_shared=args.shared, d_ffn_shared=c.F if args.shared else 0)
    ws = moe.alloc_workspace(cfg, c.k, dev)
    slots = moe.alloc_expert_slots(cfg, c.k, dev) if layer.streamed else None
    out = torch.empty((c.T, c.d), dtype=torch.int16, device=dev)
    counts = torch.zeros((nbatch, c.E), dtype=torch.int32, device=dev)
    ev_start, ev_stop = hip.create(2)
    gu, dn = moe.STAGES.index("gate_up"), moe.STAGES.index("down")
    kev = hip.create(4 * nbatch)
    profiled = not (args.shared or layer.streamed)  # kernel events on the routed layer call

    def step(i, events=None, cp=None):
        cp = layer.copies[i % len(layer.copies)] if cp is None else cp
        routing = {"expert_counts": counts[i]}
        if layer.streamed:
            moe.layer_forward_streamed(xs[i], cp["router_w"], cp["latent_down"], cp["latent_up"], layer.blob, c.k,
                                       d_ffn=c.F, expert_slots=slots, bias=bias, out=out, workspace=ws,
                                       routing=routing, packed=layer.packed, act_format=act_format)
        elif events is None or not profiled:
            moe.layer_forward(xs[i], cp["router_w"], cp["latent_down"], cp["latent_up"], layer.blob, c.k, d_ffn=c.F,
                              bias=bias, out=out, workspace=ws, routing=routing, packed=layer.packed,
                              act_format=act_format, shared_blob=layer.shared, num_shared=args.shared,
                              d_ffn_shared=c.F if args.shared else 0)
        else:
            moe.layer_forward_profiled(xs[i], cp["router_w"], cp["latent_down"], cp["latent_up"], layer.blob, c.k,
                                       events, d_ffn=c.F, bias=bias, out=out, workspace=ws, routing=routing,
                                       packed=layer.packed, act_format=act_format)

    def kernel_events(i):
        ev = moe.StageEvents()
        ev.kernel_begin[gu], ev.kernel_end[gu] = kev[4 * i], kev[4 * i + 1]
        ev.kernel_begin[dn], ev.kernel_end[dn] = kev[4 * i + 2], kev[4 * i + 3]
        return ev

    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # eager pass: warm-up, then K timed calls whose gate/up and down kernels stamp events
    for i in range(W):
        step(i, kernel_events(i))
    torch.cuda.synchronize()
    hip.record(ev_start, stream)
    for i in range(W, W + K):
        step(i, kernel_events(i))
    hip.record(ev_stop, stream)
    torch.cuda.synchronize()
    eager_ms = hip.elapsed_ms(ev_start, ev_stop)
    nan = [float("nan")] * K
    gu_ms = [hip.elapsed_ms(kev[4 * i], kev[4 * i + 1]) for i in range(W, W + K)] if profiled else nan
    dn_ms = [hip.elapsed_ms(kev[4 * i + 2], kev[4 * i + 3]) for i in range(W, W + K)] if profiled else nan

    total_ms = eager_ms
    warm_ms = None
    gu_graph_ms = dn_graph_ms = None
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
        hip.record(ev_start, stream)
        graphs[1].replay()
        hip.record(ev_stop, stream)
        torch.cuda.synchronize()
        total_ms = hip.elapsed_ms(ev_start, ev_stop)
        if profiled:
            # the same K steps captured again with the gate/up and down kernels stamping their
            # span on the device wall clock (a kernel argument, so every replay stamps it):
            # the kernels' durations in the graph the headline times
            S = moe.CLOCK_SLOTS
            clk = torch.empty((K, 2, S, 2), dtype=torch.int64, device=dev)

            def clock_events(j):
                ev = moe.StageEvents()
                ev.kernel_clock[gu] = clk[j, 0].data_ptr()
                ev.kernel_clock[dn] = clk[j, 1].data_ptr()
                return ev

            evs = [clock_events(j) for j in range(K)]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(K):
                    step(W + j, evs[j])
            for _ in range(2):
                clk[..., 0].fill_(-1)  # UINT64_MAX: lowered to the earliest block start
                clk[..., 1].fill_(0)
                g.replay()
                torch.cuda.synchronize()
            ticks = clk.cpu().numpy().view(np.uint64)
            span = ticks[..., 1].max(axis=2) - ticks[..., 0].min(axis=2)  # [K][stage]
            span_ms = span.astype(np.float64) / hip.wall_clock_khz()
            gu_graph_ms, dn_graph_ms = list(span_ms[:, 0]), list(span_ms[:, 1])
            del g
        if warm:
            # every step on batch W and dense copy 0: weights partly served from the Infinity Cache
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(K):
                    step(W, cp=layer.copies[0])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            hip.record(ev_start, stream)
            g.replay()
            hip.record(ev_stop, stream)
            torch.cuda.synchronize()
            warm_ms = hip.elapsed_ms(ev_start, ev_stop) / K
            del g
        del graphs
    ms_per_step = total_ms / K

    stages = None
    if args.breakdown and profiled:
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
    cnt = counts.cpu().numpy()[W:W + K]
    hip.destroy(kev + [ev_start, ev_stop])
    del ws, xs, out
    torch.cuda.empty_cache()
    return dict(c=c, ms_per_step=ms_per_step, eager_ms=eager_ms, warm_ms=warm_ms, gu_ms=gu_ms, dn_ms=dn_ms,
                gu_graph_ms=gu_graph_ms, dn_graph_ms=dn_graph_ms, counts=cnt, bias_host=bias_host, x_host=x_host,
                stages=stages, K=K, W=W)


def summarise(r, layer, args, moe):
    """Throughput, roofline of the dominant kernel, and the step against its own roofline."""
    c, K = r["c"], r["K"]
    # bytes of one gate (or up) matrix in the layout streamed (the same for the K3 shapes)
    mat_bytes = (moe.packed_expert_bytes(c.L, c.F) if layer.packed else moe.expert_bytes(c.L, c.F)) // 3
    active = (r["counts"] > 0).sum(1)
    # algorithmic bytes of the gate/up kernel per launch: gate and up codes+scales of every
    # active expert, the latent rows it reads (bf16) and the GLU rows it writes (bf16)
    gu_bytes = active * 2 * mat_bytes + c.T * c.L * 2 + c.T * c.k * c.F * 2
    # kernel durations: the device wall-clock span the kernel stamps inside a graph of the
    # timed steps, else the eager pass's events that the kernel's dispatch stamps (eager
    # launches run a few microseconds slower than the same kernels in a graph)
    in_graph = r["gu_graph_ms"] is not None
    gu_s = np.array(r["gu_graph_ms"] if in_graph else r["gu_ms"]) * 1e-3
    dn_s = np.array(r["dn_graph_ms"] if in_graph else r["dn_ms"]) * 1e-3
    # with shared experts the layer call takes no kernel events or clocks: no kernel time
    measured = bool(np.all(np.isfinite(gu_s)) and np.all(np.isfinite(dn_s)))

    def us(v):  # a kernel time in microseconds, or None when not measured
        return round(1e6 * float(v), 2) if measured else None

    def rnd(v, n):
        return round(float(v), n) if measured else None

    gu_eager_us = round(1e3 * float(np.mean(r["gu_ms"])), 2) if measured else None
    timing = ("device wall-clock span (first block start to last wave end) in a graph of the timed steps"
              if in_graph else "events stamped by the kernel's dispatch in the timed eager pass")
    if not measured:
        timing = "not measured: the layer call with shared experts takes no kernel events"
    # whole-layer algorithmic bytes: weights read (dense + active experts) + x + out + bias
    dense_bytes = (c.E * c.d + 2 * c.L * c.d) * 2
    layer_bytes = dense_bytes + active * 3 * mat_bytes + 2 * c.T * c.d * 2
    if args.shared:  # the shared experts' records (width d) are read every step too
        layer_bytes = layer_bytes + args.shared * (moe.packed_expert_bytes(c.d, c.F) if layer.packed
                                                   else moe.expert_bytes(c.d, c.F))
    if r["bias_host"] is not None:
        layer_bytes = layer_bytes + r["bias_host"].nbytes
    ms = r["ms_per_step"]
    layer_gbs = float(np.mean(layer_bytes) / (ms * 1e-3) / 1e9)
    # flops per step: bf16 router and latent projections, MXFP4 experts (model flops)
    f_bf16 = 2.0 * c.T * (c.d * c.E + 2 * c.d * c.L)
    f_fp4 = 2.0 * 3 * c.T * (c.k * c.L + args.shared * c.d) * c.F
    t_roof = max(float(np.mean(layer_bytes)) / (HBM_PEAK_GBS * 1e9),
                 f_fp4 / (FP4_PEAK_TFS * 1e12) + f_bf16 / (BF16_PEAK_TFS * 1e12))
    terms = 2 if args.act_format == "bf16" else 1
    out = {"ms_per_step": round(ms, 5), "tokens_per_s": round(c.T * K / (ms * K * 1e-3), 2),
           "eager_ms_per_step": round(r["eager_ms"] / K, 5),
           "mean_active_experts": float(np.mean(active)),
           "layer_roofline": {"t_roof_ms": round(t_roof * 1e3, 5), "frac": round(t_roof / (ms * 1e-3), 4),
                              "bound": "hbm" if np.mean(layer_bytes) / (HBM_PEAK_GBS * 1e9) >= t_roof else "mfma",
                              "bytes_per_step": int(np.mean(layer_bytes)), "flops_per_step": f_bf16 + f_fp4},
           "layer_hbm": {"achieved_GBs": round(layer_gbs, 1), "frac": round(layer_gbs / HBM_PEAK_GBS, 4)}}
    if r["warm_ms"] is not None:
        out["warm_cache_ms_per_step"] = round(r["warm_ms"], 5)
    if r["stages"] is not None:
        out["stages_us"] = r["stages"]
    if layer.streamed:
        link_bytes = active * 3 * mat_bytes
        link_gbs = float(np.mean(link_bytes) / (ms * 1e-3) / 1e9)
        out["roofline"] = {"bound": "host link", "kernel": "gather_experts_kernel (routed records, pinned host -> HBM)",
                           "achieved": round(link_gbs, 1), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                           "frac": round(link_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                           "note": "achieved = routed record bytes per step / whole step time (a lower bound on "
                                   "the link rate)", "bytes_per_step": int(np.mean(link_bytes))}
    elif c.T * c.k >= 8 * c.E:
        # many routed rows per expert: gate/up runs as a grouped GEMM on the matrix cores;
        # model flops 2 x rows x F x L per matrix against the dense FP4 peak.  The kernel
        # issues e4m3 x e2m1 MFMAs at the fp8 rate, `terms` per model product (the bf16
        # activations are split into two exact e4m3 terms), so its ceiling in model flops
        # is the fp8 peak / terms.
        flops = 2 * 2 * c.T * c.k * c.F * c.L
        tfs = flops / float(np.mean(gu_s)) / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": "gate_up (grouped MXFP4 GEMM + fp32 GLU)",
                           "achieved": rnd(tfs, 1), "peak": FP4_PEAK_TFS, "unit": "TFLOP/s",
                           "frac": rnd(tfs / FP4_PEAK_TFS, 4), "traffic": None,
                           "kernel_us": us(np.mean(gu_s)), "kernel_timing": timing,
                           "kernel_us_eager": gu_eager_us, "flops_per_launch": flops,
                           "mfma_terms_per_product": terms,
                           "issue_ceiling_TFs": FP8_PEAK_TFS / terms,
                           "frac_of_issue_ceiling": rnd(tfs * terms / FP8_PEAK_TFS, 4),
                           "down_kernel_us": us(np.mean(dn_s))}
    else:
        gbs = float(np.mean(gu_bytes / gu_s) / 1e9)
        dn_bytes = active * mat_bytes + c.T * c.k * c.F * 2 + c.T * c.L * 2
        out["roofline"] = {"bound": "hbm", "kernel": "gate_up (MXFP4 gate/up GEMV + fp32 GLU)",
                           "achieved": rnd(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": rnd(gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(c.name, layer.packed),
                           "kernel_us": us(np.mean(gu_s)), "kernel_timing": timing,
                           "kernel_us_eager": gu_eager_us,
                           "bytes_per_launch": int(np.mean(gu_bytes)),
                           "down_kernel_us": us(np.mean(dn_s)),
                           "down_GBs": rnd(np.mean(dn_bytes / dn_s) / 1e9, 1)}
    return out


def cpu_baseline(layer, runs, budget):
    """The C oracle timed on the host: one core on the headline workload's tokens, the same
    on all cores (token shards side by side), and prefill tokens (extrapolated)."""
    import oracle

    model, ncpu = host_info()
    cores = max(1, min(16, ncpu))
    d = layer.dense
    out = {"kind": "oracle", "cpu_model": model, "nproc": ncpu}

    def rate(r, threads, seconds, first=0):
        c = r["c"]
        xb = np.ascontiguousarray(r["x_host"].reshape(-1, c.d))
        n, t1 = 0, time.time()
        while True:
            toks = [(first + n + i) % xb.shape[0] for i in range(threads)]
            bias = r["bias_host"]
            if bias is not None and bias.ndim == 2:  # per-token bias rows of the batch the tokens come from
                bias = np.ascontiguousarray(bias[[t % c.T for t in toks]])
                xs = np.ascontiguousarray(xb[toks])
                oracle.layer_forward(xs, d["router_w"], d["latent_down"], d["latent_up"], layer.blob_host, c.k,
                                     c.L, c.F, bias=bias, threads=threads)
            else:
                oracle.layer_forward(xb, d["router_w"], d["latent_down"], d["latent_up"], layer.blob_host, c.k,
                                     c.L, c.F, bias=bias, tokens=toks, threads=threads)
            n += threads
            if time.time() - t1 >= seconds:
                break
        return n, time.time() - t1

    head = runs[0]
    n, dt = rate(head, 1, budget)
    out.update({"value": round(n / dt, 4), "unit": "tokens/s", "cores": 1,
                "sample": f"{n} tokens of the {head['c'].name} workload, whole layer one token at a time "
                          f"(single-threaded C oracle, fp64 sums, exact router), {dt:.1f} s"})
    n, dt = rate(head, cores, budget / 2, first=1)
    out["all_cores"] = {"value": round(n / dt, 4), "unit": "tokens/s", "cores": cores,
                        "sample": f"{n} tokens, {cores} token shards of the single-threaded oracle side by side, "
                                  f"{dt:.1f} s"}
    for r in runs[1:]:
        n, dt = rate(r, cores, budget / 2)
        out[r["c"].name] = {"value": round(n / dt, 4), "unit": "tokens/s", "cores": cores, "extrapolated": True,
                            "sample": f"{n} of the {r['c'].T} tokens of one {r['c'].name} batch (tokens are "
                                      f"independent in this layer, so the rate extrapolates to the whole batch), "
                                      f"{cores} shards side by side, {dt:.1f} s"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode1", choices=["decode1", "decode64", "prefill4k", "prefill32k", "tiny"])
    ap.add_argument("--prefill", action=argparse.BooleanOptionalAction, default=True,
                    help="with --config decode1, also measure prefill4k on the same layer (default)")
    ap.add_argument("--prefill-steps", type=int, default=20)
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
    if args.experts_in == "host" and args.shared:
        raise SystemExit("--experts-in host runs the routed layer only (no --shared)")

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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = HipEvents()
    layer = Layer(c, args, torch, moe, synth, dev)
    log(f"[bench] {c.name}: T={c.T}, {K} timed steps after {W} warm-up steps")
    runs = [run_config(c, layer, args, K, W, torch, moe, synth, dev, hip, warm=c.name == "decode1")]
    head = summarise(runs[0], layer, args, moe)
    log(f"[bench] {c.name}: {head['ms_per_step'] * 1e3:.1f} us per step")
    extra = {}
    if args.prefill and c.name == "decode1":
        p = synth.CONFIGS["prefill4k"]
        log(f"[bench] prefill4k on the same layer: {args.prefill_steps} timed steps")
        runs.append(run_config(p, layer, args, args.prefill_steps, 2, torch, moe, synth, dev, hip))
        s = summarise(runs[1], layer, args, moe)
        log(f"[bench] prefill4k: {s['ms_per_step']:.2f} ms per step")
        extra["prefill4k"] = dict(workload=f"{p.name}: {p.description}", steps=args.prefill_steps, warmup=2, **s)

    cpu = cpu_baseline(layer, runs, args.cpu_baseline_seconds) if args.cpu_baseline_seconds > 0 else None

    ms = head["ms_per_step"]
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms,
        "timing": ("one replay of a HIP graph holding the K steps (each on its own token batch)" if args.graph
                   else "eager calls"),
        "eager_ms_per_step": head["eager_ms_per_step"],
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
                   "dense_weight_copies": len(layer.copies), "mean_active_experts": head["mean_active_experts"],
                   "shared_experts": args.shared,
                   "expert_layout": "packed by moe_pack_experts at load" if layer.packed else "checkpoint records",
                   "experts_in": "pinned host memory, routed records fetched per step" if layer.streamed else "HBM"},
        "roofline": head["roofline"],
        "layer_roofline": head["layer_roofline"],
        "layer_hbm": head["layer_hbm"],
        "cpu_baseline": cpu,
    }
    for key in ("warm_cache_ms_per_step", "stages_us"):
        if key in head:
            result[key] = head[key]
    result.update(extra)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
