"""GPU grouped dgrad vs the oracle: out[p] = g[p] @ W_e on the packed stacks, per-row bound on
the fp32 output (8e-3 * ||row||_2 / sqrt(K) + 1e-3), bf16 output the RNE of the fp32 one."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, assert_out_is_rne_of_f32, assert_rows_within_tolerance, dev_bf16, gpu_pack, host
from moe_inputs import f32_to_bf16_bits
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


def _problem(fmt, E, N, K, counts, seed):
    rng = np.random.default_rng(seed)
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((E, N, K))).astype(np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    g = f32_to_bf16_bits(rng.standard_normal((int(offsets[-1]), N)).astype(np.float32))
    return w, g, offsets


def _check(e4b, fmt, E, N, K, counts, seed=0):
    w, g, offsets = _problem(fmt, E, N, K, counts, seed)
    packed, scales = gpu_pack(e4b, fmt, dev_bf16(w))
    out32, out = e4b.e4b_grouped_dgrad(fmt, dev_bf16(g), packed, scales,
                                       torch.from_numpy(offsets).to(DEV), out=True)
    torch.cuda.synchronize()
    op, os_ = (onf4 if fmt == "nf4" else omx).quantize_pack(w)
    ref = omoe.dgrad(fmt, op, os_, g, offsets)
    o32 = host(out32)
    assert np.all(np.isfinite(o32))
    if len(ref):
        assert_rows_within_tolerance(o32, ref, f"{fmt} E={E} N={N} K={K}")
    assert_out_is_rne_of_f32(host(out), o32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("E,N,K,counts", [
    (1, 64, 64, [1]),                          # one row, one step, partial column tile
    (3, 128, 256, [130, 0, 257]),              # an empty expert, ragged row tiles
    (4, 512, 320, [5, 128, 129, 1]),           # K not a multiple of 256
    (2, 2048, 768, [300, 77]),                 # the decode layer's down shape
])
def test_dgrad_shapes(e4b, fmt, E, N, K, counts):
    _check(e4b, fmt, E, N, K, counts, seed=E + N + K)


def test_dgrad_empty_batch(e4b):
    _check(e4b, "nf4", 3, 64, 128, [0, 0, 0])


def test_dgrad_is_deterministic(e4b):
    w, g, offsets = _problem("nf4", 4, 256, 512, [100, 200, 0, 57], 7)
    packed, scales = gpu_pack(e4b, "nf4", dev_bf16(w))
    args = (dev_bf16(g), packed, scales, torch.from_numpy(offsets).to(DEV))
    a, _ = e4b.e4b_grouped_dgrad("nf4", *args)
    b, _ = e4b.e4b_grouped_dgrad("nf4", *args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# Full-size shapes of the layers bench.py times the dgrad on: rows grouped by the oracle's
# routing of the workload's seeded logits, random packed bytes and block scales (every byte
# holds two valid codes), seeded bf16 N(0, 1) gradients.  The oracle decodes only the experts
# of the sampled rows: the first and last row of each sampled expert, rows on both sides of a
# 256-row tile boundary, and random ones.
FULL_CASES = [
    ("mixtral_nf4_prefill", "down"),
    ("mixtral_nf4_prefill", "gate_up"),
    ("mxfp4_moe", "down"),
]


@pytest.mark.parametrize("name,which", FULL_CASES, ids=[f"{n}-{w}" for n, w in FULL_CASES])
def test_dgrad_full_size_sampled_rows(e4b, name, which):
    from moe_inputs import WORKLOADS, make_logits
    from oracle import route as oroute

    wl = WORKLOADS[name]
    N, K = (wl.H, wl.I) if which == "down" else (2 * wl.I, wl.H)
    _, _, counts, offsets, _ = oroute.route(make_logits(wl), wl.k)
    offsets = np.asarray(offsets, np.int32)
    S = int(offsets[-1])
    rng = np.random.default_rng(1000 + FULL_CASES.index((name, which)))
    if wl.fmt == "nf4":
        packed = rng.integers(0, 256, (wl.E, N, K // 2), dtype=np.uint8)
        scales = (0.01 + 0.05 * rng.random((wl.E, N, K // 64))).astype(np.float32)
    else:
        packed = rng.integers(0, 256, (wl.E, N, K // 32, 16), dtype=np.uint8)
        scales = rng.integers(118, 125, (wl.E, N, K // 32), dtype=np.uint8)
    g = f32_to_bf16_bits(rng.standard_normal((S, N), dtype=np.float32))
    out32, _ = e4b.e4b_grouped_dgrad(wl.fmt, dev_bf16(g), torch.from_numpy(packed).to(DEV),
                                     torch.from_numpy(scales).to(DEV),
                                     torch.from_numpy(offsets).to(DEV))
    torch.cuda.synchronize()
    busy = [e for e in range(wl.E) if counts[e] > 0]
    experts = sorted({busy[0], busy[-1], busy[len(busy) // 2]})
    rows = []
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        cand = [lo, hi - 1, lo + 255, lo + 256, *rng.integers(lo, hi, 2).tolist()]
        rows += [r for r in cand if lo <= r < hi]
    rows = np.unique(np.asarray(rows, np.int64))
    got = host(out32)[rows]
    assert np.all(np.isfinite(host(out32)))
    ref = np.zeros((len(rows), K))
    for e in experts:
        sel = (rows >= offsets[e]) & (rows < offsets[e + 1])
        if sel.any():
            one = np.array([0, int(sel.sum())], np.int32)
            ref[sel] = omoe.dgrad(wl.fmt, packed[e:e + 1], scales[e:e + 1], g[rows[sel]], one)
    assert_rows_within_tolerance(got, ref, f"{name} {which} rows {rows.tolist()}")
