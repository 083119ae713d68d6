#!/usr/bin/env python3
"""Benchmark of the 4-bit MoE expert layer on one MI355X.

One step = one pass of the whole hot path over one batch: e4b_route_permute (top-k, softmax
weights, expert-major slot order) followed by e4b_moe_forward (x conversion, tile map,
grouped gate_up GEMM + SwiGLU, grouped down GEMM + routing weight, combine) on weights that
are already packed and resident in HBM.  Inputs are the seeded synthetic tensors of
moe_inputs.py.  Prints ONE JSON line on stdout; progress goes to stderr.

The headline workload is the Mixtral-shaped NF4 prefill layer (E=8, H=4096, I=14336, top-2,
T=4096).  The same line carries, under "secondary", the skewed 64-expert prefill layer and
the 128-expert decode layer (T=64 and T=1), and a float64 CPU-oracle baseline timed on a
bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from moe_inputs import WORKLOADS, make_expert_weight, make_logits, make_x  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD published
PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, AMD published
STAGES = ["convert_x", "build_tiles", "gemm_gate_up", "gemm_down", "combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_per_weight(fmt: str) -> float:
    return 0.5 + (4.0 / 64 if fmt == "nf4" else 1.0 / 32)


class Resident:
    """Packed weights, x and logits of one workload, resident on the GPU."""

    def __init__(self, e4b, torch, wl):
        self.e4b, self.torch, self.wl = e4b, torch, wl
        dev = "cuda:0"
        t0 = time.time()
        self.x = torch.from_numpy(make_x(wl).view(np.int16)).to(dev).view(torch.bfloat16)
        self.logits = torch.from_numpy(make_logits(wl)).to(dev)
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
        self.route_ws = torch.empty(max(256, e4b.e4b_route_workspace_bytes(wl.T, wl.E, wl.k)),
                                    dtype=torch.uint8, device=dev)
        self.fwd_ws = torch.empty(e4b.e4b_moe_workspace_bytes(wl.fmt, wl.E, wl.H, wl.I, wl.T, wl.k),
                                  dtype=torch.uint8, device=dev)
        self.out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] {wl.name}: resident in {time.time() - t0:.1f}s (pack {self.pack_s * 1e3:.1f} ms)")

    flags = 0

    def step(self, events=None):
        wl = self.wl
        ids, w, off, slots = self.e4b.e4b_route_permute(self.logits, wl.k, ws=self.route_ws)
        gp, gs = self.packed["gate_up"]
        dp, ds = self.packed["down"]
        self.e4b.e4b_moe_forward(wl.fmt, self.x, gp, gs, dp, ds, w, off, slots, wl.k, out=self.out,
                                 ws=self.fwd_ws, stage_events=events, path=self.flags)
        return off

    def active_experts(self) -> int:
        off = self.step().cpu().numpy()
        return int(np.count_nonzero(np.diff(off)))


def measure(e4b, torch, res: Resident, steps: int, warmup: int, flush_bytes: int = 0):
    """Time `steps` route+forward steps.  Per-stage kernel times come from HIP events the
    library records on the stream it launches on.  With flush_bytes > 0, a buffer of that
    size is overwritten before each step (outside the events) so weights come from HBM."""
    wl = res.wl
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0") if flush_bytes else None
    for _ in range(warmup):
        res.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for row in ev:
        for e in row:
            e.record()  # create the underlying hipEvent_t
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_begin.record()
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        step_ev[i][0].record()
        res.step(ev[i])
        step_ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    stage_ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(5)] for i in range(steps)])
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])
    total_ms = t_begin.elapsed_time(t_end)
    return {
        "ms_per_step": float(total_ms / steps) if flush is None else float(np.mean(step_ms)),
        "step_ms_median": float(np.median(step_ms)),
        "step_ms_p10": float(np.percentile(step_ms, 10)),
        "step_ms_p90": float(np.percentile(step_ms, 90)),
        "stage_ms": {s: float(np.mean(stage_ms[:, j])) for j, s in enumerate(STAGES)},
        "wall_s": wall,
    }


def roofline(wl, n_active: int, m: dict, counters: dict | None):
    """Roofline entry for the dominant kernel of the step."""
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
        abytes = 2.0 * S * wl.I + 4.0 * S * wl.H              # h read, weighted y written
    mean_rows = S / wl.E
    if mean_rows < 16:  # bandwidth-bound small-M streaming
        achieved = (wbytes + abytes) / t / 1e9
        entry = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops / t / 1e12
        entry = {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": achieved / PEAK_F16_MFMA_TFLOPS}
    entry["kernel"] = stage
    entry["kernel_ms"] = m["stage_ms"][stage]
    entry["algorithmic_bytes"] = wbytes + abytes
    entry["algorithmic_flops"] = flops
    entry["traffic"] = None
    if counters and counters.get(stage):
        entry["traffic"] = counters[stage]
    return entry


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("moe.hip", "e4b_device.h"):
        with open(os.path.join(ROOT, "bit_quantized_mixture_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_counters(workload: str) -> dict:
    """HBM traffic per launch measured with rocprofv3 counters (profiles/hbm_traffic.txt),
    used only if the kernel sources are unchanged since the counters were taken."""
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


def cpu_baseline(wl, threads_note: str):
    """The float64 oracle on a bounded sample of the workload: the rows routed to expert 0.
    Timed: oracle routing of all T tokens, decode of expert 0's gate_up and down slices,
    the float64 SwiGLU MLP on its rows and their weighted accumulation.  Scaled to tokens/s
    as (rows of expert 0 / k) / time, i.e. the rate at which the whole layer would run if
    every expert cost the same."""
    from oracle import moe as omoe
    from oracle import mxfp4 as omx
    from oracle import nf4 as onf4
    from oracle import route as oroute
    q = onf4 if wl.fmt == "nf4" else omx
    gp, gs = q.quantize_pack(make_expert_weight(wl, "gate_up", 0)[None])
    dp, ds = q.quantize_pack(make_expert_weight(wl, "down", 0)[None])
    x_bits = make_x(wl)
    logits = make_logits(wl)
    t0 = time.perf_counter()
    ids, w, counts, offsets, slots = oroute.route(logits, wl.k)
    seg = slots[offsets[0]:offsets[1]]
    tok, j = seg // wl.k, seg % wl.k
    x = omoe.bf16_bits_to_f64(x_bits[tok])
    y = omoe.expert_mlp(x, omoe.decode_expert(wl.fmt, gp, gs, 0), omoe.decode_expert(wl.fmt, dp, ds, 0))
    out = np.zeros((wl.T, wl.H))
    np.add.at(out, tok, w[tok, j][:, None] * y)
    dt = time.perf_counter() - t0
    rows = len(seg)
    return {"value": (rows / wl.k) / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{wl.name}: the {rows} rows routed to expert 0 (of {wl.T * wl.k}); oracle routing of "
                      f"all {wl.T} tokens + decode of expert 0 + float64 SwiGLU MLP + weighted accumulate; "
                      f"{dt:.1f} s; {threads_note}",
            "seconds": dt}


def blas_threads() -> str:
    try:
        from threadpoolctl import threadpool_info
        info = [f"{d.get('internal_api')}:{d.get('num_threads')}" for d in threadpool_info()]
        return "BLAS threads " + ",".join(info)
    except Exception:  # pragma: no cover
        return "BLAS threads unknown"


def workload_report(e4b, torch, wl, steps, warmup, flush=0, flags=0):
    res = Resident(e4b, torch, wl)
    res.flags = flags
    n_active = res.active_experts()
    m = measure(e4b, torch, res, steps, warmup, flush)
    rl = roofline(wl, n_active, m, load_counters(wl.name + ("" if not flush else "")))
    S = wl.T * wl.k
    ms = m["ms_per_step"]
    rep = {
        "workload": wl.name, "T": wl.T, "tokens_per_s": wl.T / (ms / 1e3), "ms_per_step": ms,
        "step_ms_median": m["step_ms_median"], "step_ms_p10": m["step_ms_p10"], "step_ms_p90": m["step_ms_p90"],
        "tflops": 6.0 * wl.H * wl.I * S / (ms / 1e3) / 1e12, "active_experts": n_active,
        "stage_ms": m["stage_ms"], "roofline": rl,
        "pack_gbs": res.pack_bytes / res.pack_s / 1e9,
        "mall_flushed": bool(flush),
    }
    del res
    torch.cuda.empty_cache()
    return rep


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_nf4_prefill", choices=list(WORKLOADS))
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flags", type=lambda v: int(v, 0), default=0,
                    help="e4b_moe_args.flags for the headline workload (path / tile override)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the layer runs on a "
              "single MI355X here; see the sharding notes in the design document.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_mixture_amd as e4b
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    wl = WORKLOADS[args.workload]
    log(f"[bench] device {torch.cuda.get_device_name(0)}; workload {wl.name}")
    main_rep = workload_report(e4b, torch, wl, args.steps, args.warmup, flags=args.flags)
    log(f"[bench] {wl.name}: {main_rep['ms_per_step']:.3f} ms/step, {main_rep['tokens_per_s']:.0f} tok/s, "
        f"{main_rep['tflops']:.1f} TFLOP/s, stages {main_rep['stage_ms']}")

    secondary = {}
    if not args.no_secondary:
        for name, T, flush in (("skewed_nf4_prefill", None, 0), ("mxfp4_moe", None, 0),
                               ("finegrained_nf4_decode", 64, 0), ("finegrained_nf4_decode", 64, 1 << 30),
                               ("finegrained_nf4_decode", 1, 0), ("finegrained_nf4_decode", 1, 1 << 30)):
            if name == wl.name and T is None:
                continue
            swl = WORKLOADS[name] if T is None else WORKLOADS[name].with_T(T)
            key = swl.name + ("" if T is None else f"_T{T}") + ("_cold" if flush else "")
            rep = workload_report(e4b, torch, swl, max(args.steps, 20), args.warmup, flush)
            secondary[key] = rep
            log(f"[bench] {key}: {rep['ms_per_step']:.4f} ms/step, {rep['tokens_per_s']:.0f} tok/s, "
                f"roofline {rep['roofline']['kernel']} {rep['roofline']['achieved']:.1f} "
                f"{rep['roofline']['unit']} ({100 * rep['roofline']['frac']:.1f}%)")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, blas_threads())
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s in {cpu['seconds']:.1f}s")

    rl = dict(main_rep["roofline"])
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
        "config": {"workload": wl.name, "fmt": wl.fmt, "E": wl.E, "H": wl.H, "I": wl.I, "k": wl.k,
                   "T": wl.T, "global_batch": wl.T, "parallelism": "single GPU"},
        "tflops": main_rep["tflops"],
        "stage_ms": main_rep["stage_ms"],
        "roofline": rl,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
