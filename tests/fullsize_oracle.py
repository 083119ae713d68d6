"""Oracle values for the full-size parity tests, computed when the tests run.

Test infrastructure: calls only oracle/ and the seeded generators of moe_inputs.py, never the
HIP library.  Every expert a checked token is routed to is packed by the oracle (in parallel
threads, one expert slice per task), then the float64 forward (the definition) and the
dequantise-to-bf16 comparator of the fidelity claim are evaluated on the checked tokens, each
over a partition of the experts in parallel threads, the partial outputs summed.

Which tokens are checked:
* "all"   every token of the batch;
* "tiles" the tokens of the first and last sorted row of every row tile the MFMA-tile path
          cuts (per expert, rows in tiles of bm = 256 when the mean routed rows per expert is
          at least 512, else 128; a last piece of at most bm / 4 rows cut into 16-row tail
          tiles instead), plus the middle row of every tail tile.  This covers the first and
          last row of every active expert, every tile boundary and every tail tile.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from moe_inputs import make_bias, make_expert_weight, make_logits, make_x
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nf4 as onf4
from oracle import route as oroute

THREADS = max(1, min(8, len(os.sched_getaffinity(0))))

_cache: dict = {}


def _packed(wl, experts):
    """Oracle-packed gate_up and down slices, dicts keyed by expert; cached per workload."""
    if _cache.get("name") != wl.name:
        _cache.clear()
        _cache.update(name=wl.name, gp={}, gs={}, dp={}, ds={})
    q = onf4 if wl.fmt == "nf4" else omx
    todo = [(e, w) for e in sorted(experts) for w in ("gate_up", "down")
            if e not in _cache["gp" if w == "gate_up" else "dp"]]

    def job(item):
        e, which = item
        return item, q.quantize_pack(make_expert_weight(wl, which, e))

    with ThreadPoolExecutor(THREADS) as ex:
        for (e, which), (p, s) in ex.map(job, todo):
            if which == "gate_up":
                _cache["gp"][e], _cache["gs"][e] = p, s
            else:
                _cache["dp"][e], _cache["ds"][e] = p, s
    return _cache["gp"], _cache["gs"], _cache["dp"], _cache["ds"]


def tile_rows(wl, offsets) -> np.ndarray:
    """Sorted rows at the boundaries of the MFMA-tile path's row tiles and tail tiles."""
    S = wl.T * wl.k
    bm = 256 if S / wl.E >= 512 else 128
    tail = bm // 4
    rows = []
    for e in range(wl.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        cnt = hi - lo
        if cnt == 0:
            continue
        nfull, rem = divmod(cnt, bm)
        split = 0 < rem <= tail
        nmain = nfull if split else -(-cnt // bm)
        for i in range(nmain):
            a = lo + i * bm
            rows += [a, min(a + bm, hi) - 1]
        if split:
            for a in range(lo + nfull * bm, hi, 16):
                b = min(a + 16, hi) - 1
                rows += [a, (a + b) // 2, b]
    return np.unique(np.asarray(rows, np.int64))


def routed(wl):
    """Oracle routing of the whole batch: ids, weights (float64), counts, offsets, slots."""
    return oroute.route(make_logits(wl), wl.k)


def checked_tokens(wl, mode: str, offsets, slots) -> np.ndarray:
    if mode == "all":
        return np.arange(wl.T, dtype=np.int64)
    if mode == "tiles":
        return np.unique(np.asarray(slots, np.int64)[tile_rows(wl, offsets)] // wl.k)
    raise ValueError(mode)


def expected(wl, tokens, ids, w, variant: bool):
    """(float64 oracle output, float64 dequantise-to-bf16 comparator output) [len(tokens), H]."""
    experts = sorted(int(e) for e in np.unique(ids[tokens]))
    gp, gs, dp, ds = _packed(wl, experts)
    x_bits = make_x(wl)
    kw = {}
    if variant:
        kw = dict(act="clamped_glu", interleaved=True,
                  b_gu=make_bias(wl, "gate_up").astype(np.float64),
                  b_dn=make_bias(wl, "down").astype(np.float64))
    groups = [set(experts[i::THREADS]) for i in range(min(THREADS, len(experts)))]

    def part(args):
        fn, grp = args
        return fn(wl.fmt, x_bits, gp, gs, dp, ds, ids, w, tokens, experts=grp, **kw)

    with ThreadPoolExecutor(THREADS) as ex:
        ref = sum(ex.map(part, [(omoe.forward, g) for g in groups]))
        cmp_ = sum(ex.map(part, [(omoe.forward_dequant_bf16, g) for g in groups]))
    return ref, cmp_
