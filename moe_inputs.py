"""Seeded synthetic inputs for the 4-bit MoE layer (shared by tests, bench and smoke).

This module only draws random numbers and rounds them to the storage dtype the layer
consumes (bf16, stored as uint16 bit patterns).  It contains none of the layer's
arithmetic: no quantisation, routing, matmul or activation.  Both the HIP path and the
CPU oracle receive the arrays produced here.

Recipe (one generator stream per tensor and per expert, so experts can be drawn one at a
time):  ``rng(tid, e) = numpy.random.default_rng(SeedSequence([seed, tid, e]))`` with
tid 0 = x, 1 = router logits, 2 = gate_up, 3 = down, 4 = gate_up bias, 5 = down bias.

* x      = bf16_rne(N(0, 1) float32 draws), shape [T, H]
* W      = bf16_rne(0.02 * N(0, 1) float32 draws), per expert, shape [N, K]
           (gate_up: N = 2I, K = H; down: N = H, K = I)
* logits = N(0, 1) float32 draws, shape [T, E]; the skewed workload adds
           float32(2 * ln(w_r)) with w_r = r^-1.2 / sum_{r'=1..E} r'^-1.2, rank r = e + 1.
* biases (expert variant only) = float32(0.02 * N(0, 1) float32 draws): gate_up [E, 2I],
           down [E, H], one stream per tensor.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TID_X, TID_LOGITS, TID_GATE_UP, TID_DOWN, TID_B_GU, TID_B_DN = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str          # "nf4", "mxfp4" or "int4" (int4-b32)
    E: int
    H: int
    I: int
    k: int
    T: int
    zipf_s: float = 0.0   # 0 = plain N(0,1) logits
    seed: int = 0

    @property
    def S(self) -> int:
        return self.T * self.k

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["workload"] = d.pop("name")
        return d


# The five workloads the layer is specified and measured on.
WORKLOADS = {
    "tiny_nf4": Workload("tiny_nf4", "nf4", E=8, H=256, I=512, k=2, T=64),
    "mixtral_nf4_prefill": Workload("mixtral_nf4_prefill", "nf4", E=8, H=4096, I=14336, k=2, T=4096),
    "finegrained_nf4_decode": Workload("finegrained_nf4_decode", "nf4", E=128, H=2048, I=768, k=8, T=64),
    "mxfp4_moe": Workload("mxfp4_moe", "mxfp4", E=32, H=2880, I=2880, k=4, T=2048),
    "skewed_nf4_prefill": Workload("skewed_nf4_prefill", "nf4", E=64, H=4096, I=1536, k=8, T=16384,
                                   zipf_s=1.2),
}
DECODE_TOKENS = (1, 4, 16, 64)

# Stacks for the int4-b32 decode GEMV (gate_up-shaped, N = 2I, K = H): the fine-grained decode
# layer's experts, and one dense [14336, 4096] matrix at M = 1 (one expert, every token routed
# to it).
INT4_WORKLOADS = {
    "finegrained_int4_decode": Workload("finegrained_int4_decode", "int4", E=128, H=2048, I=768, k=8, T=64),
    "dense_int4_decode": Workload("dense_int4_decode", "int4", E=1, H=4096, I=7168, k=1, T=1),
}


def _rng(seed: int, tid: int, e: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tid, e]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_x(wl: Workload) -> np.ndarray:
    """x bf16 bits [T, H]."""
    return f32_to_bf16_bits(_rng(wl.seed, TID_X).standard_normal((wl.T, wl.H), dtype=np.float32))


def make_logits(wl: Workload) -> np.ndarray:
    """Router logits float32 [T, E]."""
    lg = _rng(wl.seed, TID_LOGITS).standard_normal((wl.T, wl.E), dtype=np.float32)
    if wl.zipf_s:
        r = np.arange(1, wl.E + 1, dtype=np.float64)
        w = r ** (-wl.zipf_s)
        w = w / w.sum()
        lg = lg + (2.0 * np.log(w)).astype(np.float32)[None, :]
    return lg.astype(np.float32)


def make_expert_weight(wl: Workload, which: str, e: int) -> np.ndarray:
    """One expert's bf16 weight bits: gate_up [2I, H] or down [H, I]."""
    if which == "gate_up":
        tid, shape = TID_GATE_UP, (2 * wl.I, wl.H)
    elif which == "down":
        tid, shape = TID_DOWN, (wl.H, wl.I)
    else:
        raise ValueError(which)
    g = _rng(wl.seed, tid, e).standard_normal(shape, dtype=np.float32)
    g *= np.float32(0.02)
    return f32_to_bf16_bits(g)


def make_bias(wl: Workload, which: str) -> np.ndarray:
    """float32 biases of the expert variant: gate_up [E, 2I] or down [E, H]."""
    if which == "gate_up":
        tid, shape = TID_B_GU, (wl.E, 2 * wl.I)
    elif which == "down":
        tid, shape = TID_B_DN, (wl.E, wl.H)
    else:
        raise ValueError(which)
    g = _rng(wl.seed, tid).standard_normal(shape, dtype=np.float32)
    g *= np.float32(0.02)
    return g


def make_weights(wl: Workload, which: str, experts=None, threads: int = 8) -> np.ndarray:
    """Stacked bf16 bits [len(experts), N, K] (all experts by default)."""
    experts = list(range(wl.E)) if experts is None else list(experts)
    if len(experts) == 0:
        n, k = (2 * wl.I, wl.H) if which == "gate_up" else (wl.H, wl.I)
        return np.zeros((0, n, k), np.uint16)
    first = make_expert_weight(wl, which, experts[0])
    out = np.empty((len(experts),) + first.shape, np.uint16)
    out[0] = first

    def fill(i):
        out[i] = make_expert_weight(wl, which, experts[i])

    if len(experts) > 1:
        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(fill, range(1, len(experts))))
    return out


def bytes_bf16(shape) -> int:
    return 2 * math.prod(shape)
