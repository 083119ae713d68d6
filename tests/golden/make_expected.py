#!/usr/bin/env python3
"""Writes tests/golden/expected_<case>.npz: oracle outputs of sampled tokens of each full-size
workload, for tests/test_gpu_fullsize.py.

Calls only oracle/ (and the seeded input generators of moe_inputs.py): route all T tokens,
pick the sampled tokens, pack with the oracle every expert those tokens are routed to, and
run the float64 forward on those tokens.  Stored per case: the sampled token indices, their
routed expert ids and weights (oracle routing), and the float64 outputs [n, H].

Usage: python tests/golden/make_expected.py [case ...]   (all cases by default)
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from moe_inputs import WORKLOADS, make_bias, make_expert_weight, make_logits, make_x  # noqa: E402
from oracle import moe as omoe  # noqa: E402
from oracle import mxfp4 as omx  # noqa: E402
from oracle import nf4 as onf4  # noqa: E402
from oracle import route as oroute  # noqa: E402

# (case name, workload, T override or None); a "_clamped_glu" case is the expert variant
# (interleaved gate/up rows, clamped GLU, seeded biases of moe_inputs.make_bias)
CASES = [
    ("mixtral_nf4_prefill", "mixtral_nf4_prefill", None),
    ("finegrained_nf4_decode_T1", "finegrained_nf4_decode", 1),
    ("finegrained_nf4_decode_T4", "finegrained_nf4_decode", 4),
    ("finegrained_nf4_decode_T16", "finegrained_nf4_decode", 16),
    ("finegrained_nf4_decode_T64", "finegrained_nf4_decode", 64),
    ("mxfp4_moe", "mxfp4_moe", None),
    ("skewed_nf4_prefill", "skewed_nf4_prefill", None),
    ("mxfp4_moe_clamped_glu", "mxfp4_moe", None),
]
N_SAMPLE = 6


def sample_tokens(T: int, seed: int = 1234) -> np.ndarray:
    """The first and last token and random others (all tokens when T <= N_SAMPLE)."""
    if T <= N_SAMPLE:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), N_SAMPLE - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid])).astype(np.int64)


def expected(case: str, name: str, T):
    wl = WORKLOADS[name] if T is None else WORKLOADS[name].with_T(T)
    q = onf4 if wl.fmt == "nf4" else omx
    x_bits = make_x(wl)
    ids, w, counts, offsets, slots = oroute.route(make_logits(wl), wl.k)
    toks = sample_tokens(wl.T)
    gp, gs, dp, ds = {}, {}, {}, {}
    for e in np.unique(ids[toks]):
        e = int(e)
        gp[e], gs[e] = q.quantize_pack(make_expert_weight(wl, "gate_up", e))
        dp[e], ds[e] = q.quantize_pack(make_expert_weight(wl, "down", e))
    kw = {}
    if case.endswith("_clamped_glu"):
        kw = dict(act="clamped_glu", interleaved=True,
                  b_gu=make_bias(wl, "gate_up").astype(np.float64),
                  b_dn=make_bias(wl, "down").astype(np.float64))
    out = omoe.forward(wl.fmt, x_bits, gp, gs, dp, ds, ids, w, toks, **kw)
    return {"tokens": toks, "ids": ids[toks].astype(np.int32), "w": w[toks].astype(np.float64),
            "out": out}


def main(argv):
    want = set(argv) if argv else {c for c, _, _ in CASES}
    for case, name, T in CASES:
        if case not in want:
            continue
        t0 = time.time()
        d = expected(case, name, T)
        path = os.path.join(HERE, f"expected_{case}.npz")
        np.savez_compressed(path, **d)
        print(f"{case}: {len(d['tokens'])} tokens, {d['out'].shape}, {time.time() - t0:.0f}s -> {path}",
              flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
