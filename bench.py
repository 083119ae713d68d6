#!/usr/bin/env python3
"""Benchmark of the 4-bit MoE expert layer on one MI355X.

One step = one pass of the whole hot path over one batch: e4b_route_permute (top-k, softmax
weights, expert-major slot order) followed by e4b_moe_forward (x conversion, tile map,
grouped gate_up GEMM + SwiGLU, grouped down GEMM, weighted combine) on weights that are
already packed and resident in HBM.  Inputs are the seeded synthetic tensors of
moe_inputs.py.  Prints ONE JSON line on stdout; progress goes to stderr.

The headline workload is the largest prefill layer, the skewed 64-expert NF4 layer (E=64,
H=4096, I=1536, top-8, T=16384, Zipf-biased routing with 20 empty experts).  The same line
carries, under "secondary", the Mixtral-shaped NF4 prefill layer (E=8, H=4096, I=14336, top-2,
T=4096), the MXFP4 layer (also run as the MXFP4 family's expert variant: interleaved gate/up
rows, clamped GLU, per-expert biases) and the 128-expert decode layer at T = 64, 16, 4, 1 (warm,
and cold with the 256 MB Infinity Cache flushed by reading 1 GiB before every step; eager
launches with per-stage HIP events, and the same step replayed from a HIP graph; at T = 1, 4, 8
also the single-launch decode step, eager and graph-replayed), and a float64
CPU-oracle baseline timed on a bounded sample of the headline workload.  Also under
"secondary": the grouped dgrad on the Mixtral-shaped layer's packed down and gate_up stacks
with its own routing, and the int4-b32 routed decode GEMV (exact integer accumulation) on the
decode layer's gate_up stack at T = 64 and 1 and on one dense [14336, 4096] matrix at M = 1, in
GB/s of weight streaming.  "hbm_ceiling" holds the rates of a plain streaming read and a plain
copy (the library's e4b_stream_probe) and of torch's device copy, measured in the same run,
beside the published 8 TB/s.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from moe_inputs import INT4_WORKLOADS, WORKLOADS, make_bias, make_expert_weight, make_logits, make_x  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD published
PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, AMD published
STAGES = ["convert_x", "build_tiles", "gemm_gate_up", "gemm_down", "combine"]
MALL_FLUSH_BYTES = 1 << 30     # > 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_per_weight(fmt: str) -> float:
    return 0.5 + (4.0 / 64 if fmt == "nf4" else 1.0 / 32)


class Layer:
    """Packed weights of one workload, resident on the GPU (packed there by the library)."""

    def __init__(self, e4b, torch, wl):
        self.e4b, self.torch, self.wl = e4b, torch, wl
        dev = "cuda:0"
        t0 = time.time()
        self.packed = {}
        self.pack_s = 0.0
        for which, (N, K) in (("gate_up", (2 * wl.I, wl.H)), ("down", (wl.H, wl.I))):
            w = torch.empty((wl.E, N, K), dtype=torch.bfloat16, device=dev)
            for e in range(wl.E):
                w[e].copy_(torch.from_numpy(make_expert_weight(wl, which, e).view(np.int16)).view(torch.bfloat16))
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if wl.fmt == "nf4":
                self.packed[which] = e4b.e4b_pack_nf4(w)
            else:
                self.packed[which] = e4b.e4b_pack_mxfp4(w)
            b.record()
            torch.cuda.synchronize()
            self.pack_s += a.elapsed_time(b) / 1e3
            del w
        self.pack_bytes = wl.E * 3 * wl.H * wl.I * (2 + bytes_per_weight(wl.fmt))  # bf16 in, codes+scales out
        torch.cuda.synchronize()
        log(f"[bench] {wl.name}: weights resident in {time.time() - t0:.1f}s (GPU pack {self.pack_s * 1e3:.1f} ms)")


class Batch:
    """x, router logits and every output / workspace buffer of one batch size."""

    flags = 0
    variant = {}  # expert-variant keyword arguments of e4b_moe_forward (act, interleaved, biases)

    def __init__(self, layer: Layer, T: int, flags: int = 0):
        torch, e4b = layer.torch, layer.e4b
        self.layer, self.e4b = layer, e4b
        self.flags = flags
        self.wl = wl = layer.wl.with_T(T)
        dev = "cuda:0"
        self.x = torch.from_numpy(make_x(wl).view(np.int16)).to(dev).view(torch.bfloat16)
        self.logits = torch.from_numpy(make_logits(wl)).to(dev)
        self.route_out = (torch.empty((T, wl.k), dtype=torch.int32, device=dev),
                          torch.empty((T, wl.k), dtype=torch.float32, device=dev),
                          torch.empty((wl.E + 1,), dtype=torch.int32, device=dev),
                          torch.empty((T * wl.k,), dtype=torch.int32, device=dev))
        self.route_ws = torch.empty(max(256, e4b.e4b_route_workspace_bytes(T, wl.E, wl.k)),
                                    dtype=torch.uint8, device=dev)
        self.fwd_ws = torch.empty(max(256, e4b.e4b_moe_workspace_bytes(wl.fmt, wl.E, wl.H, wl.I, T, wl.k, flags)),
                                  dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, wl.H), dtype=torch.bfloat16, device=dev)

    def step(self, events=None):
        wl = self.wl
        ids, w, off, slots = self.e4b.e4b_route_permute(self.logits, wl.k, ws=self.route_ws, out=self.route_out)
        gp, gs = self.layer.packed["gate_up"]
        dp, ds = self.layer.packed["down"]
        self.e4b.e4b_moe_forward(wl.fmt, self.x, gp, gs, dp, ds, w, off, slots, wl.k, out=self.out,
                                 ws=self.fwd_ws, stage_events=events, path=self.flags, **self.variant)
        return off

    def active_experts(self) -> int:
        off = self.step().cpu().numpy()
        return int(np.count_nonzero(np.diff(off)))


def measure(torch, b: Batch, steps: int, warmup: int, flush_bytes: int = 0):
    """Time `steps` route+forward steps.  Per-stage kernel times come from HIP events the
    library records on the stream it launches on.  With flush_bytes > 0, a buffer of that
    size is read (summed) before each step, outside the events, so the weights come from HBM.
    The flush reads rather than writes: a written buffer leaves dirty lines in the caches,
    and writing them back during the step would be charged to the kernels."""
    flush = torch.zeros(flush_bytes // 4, dtype=torch.int32, device="cuda:0") if flush_bytes else None
    for _ in range(warmup):
        b.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for row in ev:
        for e in row:
            e.record()  # create the underlying hipEvent_t
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # no Python garbage collection inside the timed region (a collection that frees the
    # previous layer's tensors there stalled the launch thread by milliseconds)
    gc.collect()
    gc.disable()
    wall0 = time.perf_counter()
    t_begin.record()
    for i in range(steps):
        if flush is not None:
            flush.sum()
        step_ev[i][0].record()
        b.step(ev[i])
        step_ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    stage_ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(5)] for i in range(steps)])
    step_ms = np.array([a.elapsed_time(c) for a, c in step_ev])
    total_ms = t_begin.elapsed_time(t_end)
    return {
        "ms_per_step": float(total_ms / steps) if flush is None else float(np.mean(step_ms)),
        "step_ms_median": float(np.median(step_ms)),
        "step_ms_p10": float(np.percentile(step_ms, 10)),
        "step_ms_p90": float(np.percentile(step_ms, 90)),
        "stage_ms": {s: float(np.mean(stage_ms[:, j])) for j, s in enumerate(STAGES)},
        "wall_s": wall,
    }


def measure_graph(torch, b: Batch, steps: int):
    """The same step captured once into a HIP graph and replayed `steps` times back to back
    (no per-stage events): the step's GPU time without host launch gaps."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            b.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    c.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(c) / steps
    del g
    return ms


def roofline(wl, n_active: int, m: dict, counters: dict | None):
    """Roofline entry for the dominant kernel of the step (algorithmic work per launch over
    its mean launch time from the HIP events)."""
    S = wl.T * wl.k
    bw = bytes_per_weight(wl.fmt)
    stage = max(("gemm_gate_up", "gemm_down"), key=lambda s: m["stage_ms"][s])
    t = m["stage_ms"][stage] / 1e3
    if stage == "gemm_gate_up":
        flops = 4.0 * wl.H * wl.I * S
        wbytes = n_active * 2 * wl.I * wl.H * bw
        abytes = 2.0 * wl.T * wl.H + 2.0 * S * wl.I          # x (fp16) read, h (fp16) written
    else:
        flops = 2.0 * wl.H * wl.I * S
        wbytes = n_active * wl.H * wl.I * bw
        abytes = 2.0 * S * wl.I + 4.0 * S * wl.H              # h read, y (fp32) written
    mean_rows = S / wl.E
    if mean_rows < 16:  # bandwidth-bound small-M streaming
        achieved = (wbytes + abytes) / t / 1e9
        entry = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops / t / 1e12
        entry = {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": achieved / PEAK_F16_MFMA_TFLOPS}
    entry["traffic"] = None
    if counters and counters.get(stage):
        entry["traffic"] = counters[stage]
    entry["kernel"] = stage
    entry["kernel_ms"] = m["stage_ms"][stage]
    entry["algorithmic_bytes"] = wbytes + abytes
    entry["algorithmic_flops"] = flops
    return entry


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("moe.hip", "gemv.hip", "e4b_device.h"):
        with open(os.path.join(ROOT, "bit_quantized_mixture_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_counters(workload: str) -> dict:
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (profiles/hbm_traffic.txt,
    already scaled by the copy-kernel calibration), used only while the kernel sources are
    the ones the counters were taken on.  `workload` is the workload name, with _T<T> appended
    for a batch size other than the workload's own."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    out = {}
    if not os.path.exists(path):
        return out
    sha = kernel_source_sha()
    with open(path) as f:
        for ln in f:
            p = ln.split()
            if len(p) == 5 and not ln.startswith("#") and p[0] == workload and p[2] == sha:
                out[p[1]] = float(p[3]) + float(p[4])
    return out


def cpu_baseline(wl, threads_note: str, min_s: float = 12.0, max_reps: int = 40):
    """The float64 oracle on a bounded sample of the workload: the rows routed to expert 0.
    Packing expert 0's two weight slices with the oracle is timed on its own (elements/s).
    The forward sample -- oracle routing of all T tokens, decode of expert 0's gate_up and
    down slices, the float64 SwiGLU MLP on its rows and their weighted accumulation -- is
    repeated until it has run at least `min_s` seconds, and scaled to tokens/s as
    (rows of expert 0 / k) * repetitions / time, i.e. the rate at which the whole layer would
    run if every expert cost the same."""
    from oracle import moe as omoe
    from oracle import mxfp4 as omx
    from oracle import nf4 as onf4
    from oracle import route as oroute
    q = onf4 if wl.fmt == "nf4" else omx
    g_bits, d_bits = make_expert_weight(wl, "gate_up", 0), make_expert_weight(wl, "down", 0)
    t0 = time.perf_counter()
    gp, gs = q.quantize_pack(g_bits[None])
    dp, ds = q.quantize_pack(d_bits[None])
    pack_s = time.perf_counter() - t0
    x_bits = make_x(wl)
    logits = make_logits(wl)
    reps, rows = 0, 0
    t0 = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_s):
        ids, w, counts, offsets, slots = oroute.route(logits, wl.k)
        seg = slots[offsets[0]:offsets[1]]
        tok, j = seg // wl.k, seg % wl.k
        x = omoe.bf16_bits_to_f64(x_bits[tok])
        y = omoe.expert_mlp(x, omoe.decode_expert(wl.fmt, gp, gs, 0), omoe.decode_expert(wl.fmt, dp, ds, 0))
        out = np.zeros((wl.T, wl.H))
        np.add.at(out, tok, w[tok, j][:, None] * y)
        rows = len(seg)
        reps += 1
    dt = time.perf_counter() - t0
    n_el = g_bits.size + d_bits.size
    return {"value": (rows / wl.k) * reps / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{wl.name}: the {rows} rows routed to expert 0 (of {wl.T * wl.k}); oracle routing of "
                      f"all {wl.T} tokens + decode of expert 0 + float64 SwiGLU MLP + weighted accumulate, "
                      f"{reps} repetitions in {dt:.1f} s; {threads_note}",
            "seconds": dt,
            "pack_elements_per_s": n_el / pack_s,
            "pack_sample": f"oracle {wl.fmt} packing of expert 0's gate_up and down ({n_el} elements) in {pack_s:.1f} s"}


def blas_threads() -> str:
    try:
        from threadpoolctl import threadpool_info
        info = [f"{d.get('internal_api')}:{d.get('num_threads')}" for d in threadpool_info()]
        return "BLAS threads " + ",".join(info)
    except Exception:  # pragma: no cover
        return "BLAS threads unknown"


def expert_variant(torch, wl) -> dict:
    """e4b_moe_forward keywords of the MXFP4 family's expert variant: gate/up rows read as
    interleaved, clamped GLU, the seeded biases of moe_inputs.make_bias."""
    return dict(act="clamped_glu", interleaved=True,
                b_gu=torch.from_numpy(make_bias(wl, "gate_up")).to("cuda:0"),
                b_dn=torch.from_numpy(make_bias(wl, "down")).to("cuda:0"))


def batch_report(torch, layer: Layer, T: int, steps: int, warmup: int, flush: int = 0, flags: int = 0,
                 graph: bool = False, variant: dict | None = None, counters: bool = True):
    b = Batch(layer, T, flags)
    b.variant = variant or {}
    wl = b.wl
    n_active = b.active_experts()
    m = measure(torch, b, steps, warmup, flush)
    # the counters were taken at each workload's own T; other batch sizes get none; the expert
    # variant has rows of its own
    key = wl.name if wl.T == WORKLOADS[wl.name].T else f"{wl.name}_T{wl.T}"
    if b.variant:
        key += "_clamped_glu"
    rl = roofline(wl, n_active, m, None if (flush or not counters) else load_counters(key))
    S = wl.T * wl.k
    ms = m["ms_per_step"]
    rep = {
        "workload": wl.name, "T": wl.T, "tokens_per_s": wl.T / (ms / 1e3), "ms_per_step": ms,
        "step_ms_median": m["step_ms_median"], "step_ms_p10": m["step_ms_p10"], "step_ms_p90": m["step_ms_p90"],
        "tflops": 6.0 * wl.H * wl.I * S / (ms / 1e3) / 1e12, "active_experts": n_active,
        "stage_ms": m["stage_ms"], "roofline": rl,
        "mall_flushed": bool(flush),
    }
    if graph:
        gms = measure_graph(torch, b, max(steps, 50))
        rep["graph_ms_per_step"] = gms
        rep["graph_tokens_per_s"] = wl.T / (gms / 1e3)
    del b
    torch.cuda.empty_cache()
    return rep


def dgrad_report(torch, layer: Layer, steps: int, warmup: int) -> dict:
    """Grouped dgrad on the layer's packed stacks, with the layer's own routing: down
    (g [S, H] -> [S, I]) and gate_up (g [S, 2I] -> [S, H]); seeded bf16 N(0, 1) gradients.
    Timed with HIP events on the current stream (one launch each, after warm-up)."""
    e4b, wl = layer.e4b, layer.wl
    b = Batch(layer, wl.T)
    off = b.step()
    S = wl.T * wl.k
    g_gen = torch.Generator(device="cuda:0").manual_seed(1)
    rep = {}
    for which, N, K in (("down", wl.H, wl.I), ("gate_up", 2 * wl.I, wl.H)):
        w, sc = layer.packed[which]
        g = torch.randn((S, N), generator=g_gen, device="cuda:0").to(torch.bfloat16)
        out = torch.empty((S, K), dtype=torch.float32, device="cuda:0")
        ws = torch.empty((max(e4b.e4b_dgrad_workspace_bytes(wl.fmt, wl.E, N, K, S), 256),),
                         dtype=torch.uint8, device="cuda:0")
        run = lambda: e4b.e4b_grouped_dgrad(wl.fmt, g, w, sc, off, out_f32=out, ws=ws)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            run()
        t1.record()
        torch.cuda.synchronize()
        gc.enable()
        ms = t0.elapsed_time(t1) / steps
        flops = 2.0 * S * N * K
        tf = flops / (ms / 1e3) / 1e12
        rep[which] = {"ms": ms, "tflops": tf, "frac_of_mfma_peak": tf / PEAK_F16_MFMA_TFLOPS,
                      "algorithmic_flops": flops, "S": S, "N": N, "K": K}
        del g, out, ws
    del b
    torch.cuda.empty_cache()
    return rep


def int4_report(torch, e4b, wl, T: int, steps: int, warmup: int) -> dict:
    """The int4-b32 routed decode GEMV on the workload's gate_up-shaped stack (seeded bf16
    weights packed on the GPU by e4b_pack_int4_b32), T tokens routed by the seeded logits.
    One call = activation quantiser + tile list + GEMV, timed with HIP events on the current
    stream.  Algorithmic bytes: the active experts' codes and scales (0.5625 B per weight),
    x (2 B per element) and the fp32 output."""
    dev = "cuda:0"
    N, K = 2 * wl.I, wl.H
    w = torch.empty((wl.E, N, K), dtype=torch.bfloat16, device=dev)
    for e in range(wl.E):
        w[e].copy_(torch.from_numpy(make_expert_weight(wl, "gate_up", e).view(np.int16)).view(torch.bfloat16))
    packed, scales = e4b.e4b_pack_int4_b32(w)
    del w
    wt = wl.with_T(T)
    x = torch.from_numpy(make_x(wt).view(np.int16)).to(dev).view(torch.bfloat16)
    _, _, off, slots = e4b.e4b_route_permute(torch.from_numpy(make_logits(wt)).to(dev), wl.k)
    out = torch.empty((T * wl.k, N), dtype=torch.float32, device=dev)
    ws = torch.empty((max(e4b.e4b_int4_gemv_workspace_bytes(wl.E, N, K, T, wl.k), 256),),
                     dtype=torch.uint8, device=dev)
    run = lambda: e4b.e4b_gemv_int4_b32(packed, scales, x, wl.k, off, slots, out=out, ws=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    active = int((torch.diff(off) > 0).sum().item())
    gc.collect()
    gc.disable()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        run()
    t1.record()
    torch.cuda.synchronize()
    gc.enable()
    ms = t0.elapsed_time(t1) / steps
    nbytes = active * N * K * 0.5625 + T * K * 2 + T * wl.k * N * 4
    gbs = nbytes / (ms / 1e3) / 1e9
    del packed, scales, x, out, ws
    torch.cuda.empty_cache()
    return {"ms": ms, "T": T, "E": wl.E, "N": N, "K": K, "k": wl.k, "active_experts": active,
            "algorithmic_bytes": nbytes, "achieved_gbs": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}


def decode_step_report(torch, layer: Layer, T: int, steps: int, warmup: int) -> dict:
    """The single-launch decode step (e4b_moe_decode_step: routing, gate_up, down and combine in
    one kernel) on the layer's packed weights at batch T, eager (HIP events on the current
    stream around each call) and replayed from a HIP graph.  Algorithmic bytes: the active
    experts' packed weights and scales, x, logits and the bf16 output."""
    e4b, wl = layer.e4b, layer.wl.with_T(T)
    dev = "cuda:0"
    x = torch.from_numpy(make_x(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(make_logits(wl)).to(dev)
    ws = torch.zeros(e4b.e4b_decode_workspace_bytes(wl.fmt, wl.E, wl.H, wl.I, T, wl.k), dtype=torch.uint8, device=dev)
    out = torch.empty((T, wl.H), dtype=torch.bfloat16, device=dev)
    gp, gs = layer.packed["gate_up"]
    dp, ds = layer.packed["down"]
    run = lambda: e4b.e4b_moe_decode_step(wl.fmt, logits, x, gp, gs, dp, ds, wl.k, out=out, ws=ws)
    ids = np.argsort(-make_logits(wl), axis=1, kind="stable")[:, :wl.k]
    active = len(np.unique(ids))
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    gc.enable()
    eager = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    graph = t0.elapsed_time(t1) / steps
    del g
    nbytes = active * 3 * wl.H * wl.I * bytes_per_weight(wl.fmt) + 2 * T * wl.H * 2 + 4 * T * wl.E
    return {"T": T, "active_experts": active, "ms_per_step": eager, "graph_ms_per_step": graph,
            "tokens_per_s": T / (eager / 1e3), "graph_tokens_per_s": T / (graph / 1e3),
            "algorithmic_bytes": nbytes, "achieved_gbs": nbytes / (eager / 1e3) / 1e9,
            "frac_of_hbm_peak": nbytes / (eager / 1e3) / 1e9 / PEAK_HBM_GBS}


def hbm_ceiling(torch, e4b, nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """Measured ceilings beside the published HBM peak, on a buffer of `nbytes` (16 times the
    256 MB Infinity Cache): the library's plain streaming read (e4b_stream_probe, 16-byte loads,
    nothing written) and plain copy (read + written bytes per second), and torch's device copy;
    each the mean of `reps` launches timed with HIP events on the current stream."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    res = {}
    for key, fn, moved in (("read_gbs", lambda: e4b.e4b_stream_probe(a), nbytes),
                           ("copy_gbs", lambda: e4b.e4b_stream_probe(a, b), 2 * nbytes),
                           ("torch_copy_gbs", lambda: b.copy_(a), 2 * nbytes)):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        res[key] = moved / (t0.elapsed_time(t1) / reps / 1e3) / 1e9
    res["bytes"] = nbytes
    res["published_gbs"] = PEAK_HBM_GBS
    del a, b
    torch.cuda.empty_cache()
    return res


def fmt_rep(key, rep):
    rl = rep["roofline"]
    s = (f"[bench] {key}: {rep['ms_per_step']:.4f} ms/step, {rep['tokens_per_s']:.0f} tok/s, "
         f"{rl['kernel']} {rl['achieved']:.1f} {rl['unit']} ({100 * rl['frac']:.1f}% of peak)")
    if "graph_ms_per_step" in rep:
        s += f", graph {rep['graph_ms_per_step']:.4f} ms/step"
    return s


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="skewed_nf4_prefill", choices=list(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=0,
                    help="batch size of the headline workload (default: the workload's own T)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="all",
                    help="comma list of secondary sections to run: dgrad, prefill (the skewed and "
                         "MXFP4 layers), int4, decode; default all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flags", type=lambda v: int(v, 0), default=0,
                    help="e4b_moe_args.flags for the headline workload (path / tile override)")
    ap.add_argument("--variant", action="store_true",
                    help="run the headline workload as the MXFP4 family's expert variant (clamped "
                         "GLU, interleaved gate/up rows, the seeded biases)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the layer runs on a "
              "single MI355X; the multi-GPU (expert- or tensor-parallel) path is not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_mixture_amd as e4b
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    wl = WORKLOADS[args.workload]
    if args.tokens:
        wl = wl.with_T(args.tokens)
    log(f"[bench] device {torch.cuda.get_device_name(0)}; workload {wl.name}, T = {wl.T}")
    layer = Layer(e4b, torch, wl)
    pack_gbs = layer.pack_bytes / layer.pack_s / 1e9
    main_rep = batch_report(torch, layer, wl.T, args.steps, args.warmup, flags=args.flags,
                            variant=expert_variant(torch, wl) if args.variant else None)
    log(fmt_rep(wl.name, main_rep) + f"; stages {main_rep['stage_ms']}")
    secondary = {}
    sections = set() if args.no_secondary else (
        {"dgrad", "prefill", "int4", "decode"} if args.secondary == "all" else set(args.secondary.split(",")))
    if "prefill" in sections and not args.flags & e4b.E4B_COMBINE_ATOMIC:
        # the same layer with the atomic scatter-combine in the down GEMM (E4B_COMBINE_ATOMIC);
        # the counters in profiles/ were taken on the ordered combine, so no traffic figure
        key = wl.name + "_atomic_combine"
        secondary[key] = batch_report(torch, layer, wl.T, args.steps, args.warmup,
                                      flags=args.flags | e4b.E4B_COMBINE_ATOMIC, counters=False)
        log(fmt_rep(key, secondary[key]) + f"; stages {secondary[key]['stage_ms']}")
    del layer
    torch.cuda.empty_cache()
    ceiling = hbm_ceiling(torch, e4b)
    log(f"[bench] HBM ceiling: read {ceiling['read_gbs']:.0f} GB/s, copy {ceiling['copy_gbs']:.0f} GB/s "
        f"(torch copy {ceiling['torch_copy_gbs']:.0f} GB/s)")

    dgrad_on = "mixtral_nf4_prefill"
    for name in ("mixtral_nf4_prefill", "skewed_nf4_prefill", "mxfp4_moe"):
        run_fwd = "prefill" in sections and name != wl.name
        run_dgrad = "dgrad" in sections and name == dgrad_on
        if not (run_fwd or run_dgrad):
            continue
        lay = Layer(e4b, torch, WORKLOADS[name])
        if run_dgrad:
            secondary[name + "_dgrad"] = dg = dgrad_report(torch, lay, max(args.steps, 10), args.warmup)
            log(f"[bench] {name} dgrad: " + ", ".join(
                f"{k} {v['ms']:.3f} ms {v['tflops']:.1f} TFLOP/s ({100 * v['frac_of_mfma_peak']:.1f}%)"
                for k, v in dg.items()))
        if run_fwd:
            secondary[name] = batch_report(torch, lay, WORKLOADS[name].T, max(args.steps, 10), args.warmup)
            log(fmt_rep(name, secondary[name]))
            if name == "mxfp4_moe":
                # the same layer as the MXFP4 family's expert variant
                wv = WORKLOADS[name]
                variant = expert_variant(torch, wv)
                key = name + "_clamped_glu"
                secondary[key] = batch_report(torch, lay, wv.T, max(args.steps, 10), args.warmup,
                                              variant=variant)
                log(fmt_rep(key, secondary[key]))
                # the gate_up on the block-scaled fp8 x fp4 instruction (E4B_MXFP4_SCALED); the
                # counters in profiles/ were taken on the default route, so no traffic figure
                key = name + "_scaled_route"
                secondary[key] = batch_report(torch, lay, wv.T, max(args.steps, 10), args.warmup,
                                              flags=e4b.E4B_MXFP4_SCALED, counters=False)
                log(fmt_rep(key, secondary[key]))
        del lay
        torch.cuda.empty_cache()
    if "int4" in sections:
        for name, T in (("finegrained_int4_decode", 64), ("finegrained_int4_decode", 1),
                        ("dense_int4_decode", 1)):
            key = f"{name}_T{T}"
            secondary[key] = r = int4_report(torch, e4b, INT4_WORKLOADS[name], T, max(args.steps, 50), args.warmup)
            log(f"[bench] {key}: {r['ms'] * 1e3:.2f} us/call, {r['achieved_gbs']:.1f} GB/s "
                f"({100 * r['frac_of_hbm_peak']:.1f}% of HBM peak), {r['active_experts']} experts")
    if "decode" in sections:
        dwl = WORKLOADS["finegrained_nf4_decode"]
        lay = Layer(e4b, torch, dwl)
        for T, flush in ((64, 0), (16, 0), (4, 0), (1, 0), (64, MALL_FLUSH_BYTES), (1, MALL_FLUSH_BYTES)):
            key = f"{dwl.name}_T{T}" + ("_cold" if flush else "")
            secondary[key] = batch_report(torch, lay, T, max(args.steps, 50), args.warmup, flush,
                                          graph=not flush)
            log(fmt_rep(key, secondary[key]))
        for T in (1, 4, 8):
            key = f"{dwl.name}_T{T}_single_launch"
            secondary[key] = r = decode_step_report(torch, lay, T, max(args.steps, 50), args.warmup)
            log(f"[bench] {key}: {r['ms_per_step']:.4f} ms/step eager, {r['graph_ms_per_step']:.4f} ms/step "
                f"graph, {r['achieved_gbs']:.0f} GB/s ({100 * r['frac_of_hbm_peak']:.1f}% of HBM peak)")
        del lay
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, blas_threads())
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s over {cpu['seconds']:.1f}s; "
            f"oracle pack {cpu['pack_elements_per_s'] / 1e6:.1f} M elements/s")

    line = {
        "metric": "MoE layer tokens/s + achieved HBM GB/s / MFMA TFLOP/s vs MI355X peak",
        "value": main_rep["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rep["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) x and logits, N(0,0.02) bf16 weights packed on the GPU)",
        "config": {"workload": wl.name + ("_clamped_glu" if args.variant else ""), "fmt": wl.fmt,
                   "E": wl.E, "H": wl.H, "I": wl.I, "k": wl.k,
                   "T": wl.T, "global_batch": wl.T, "parallelism": "single GPU"},
        "tflops": main_rep["tflops"],
        "stage_ms": main_rep["stage_ms"],
        "roofline": dict(main_rep["roofline"]),
        "cpu_baseline": cpu,
        "hbm_ceiling": ceiling,
        "gpu_pack_gbs": pack_gbs,
        "secondary": secondary,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
