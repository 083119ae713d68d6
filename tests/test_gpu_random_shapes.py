"""Seeded random shapes through every path, against the oracle: the forward (formats, paths, row
tiles, the expert variant), the grouped dgrad and the int4-b32 GEMV.  Each case draws its shape
from its own fixed seed, so the set is the same on every run; the bounds are those of the other
parity tests (per-row tolerance for the forward and dgrad, the float32 bound for int4)."""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, assert_out_is_rne_of_f32, assert_rows_within_tolerance, dev_bf16,
                         gpu_pack, host, random_layer)
from moe_inputs import f32_to_bf16_bits
from oracle import int4 as oi4
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nf4 as onf4
from oracle import route as oroute

pytestmark = pytest.mark.gpu

TILES = [0x0, 0x4, 0x8, 0xC]   # E4B_TILE_AUTO / 32 / 128 / 256 (with the MFMA path)


@pytest.mark.parametrize("case", range(16))
def test_random_forward(e4b, case):
    rng = np.random.default_rng(1000 + case)
    fmt = ("nf4", "mxfp4")[case % 2]
    E = int(rng.integers(1, 25))
    k = int(rng.integers(1, min(E, 8) + 1))
    H, I = 64 * int(rng.integers(1, 17)), 64 * int(rng.integers(1, 13))
    T = int(rng.integers(1, 400))
    path = int(rng.integers(0, 3))
    flags = path | (TILES[int(rng.integers(0, 4))] if path == 1 else 0)
    variant = case % 3 == 0
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=2000 + case)
    kw = {}
    if variant:
        kw = dict(act="clamped_glu", interleaved=True,
                  b_gu=(0.02 * rng.standard_normal((E, 2 * I))).astype(np.float32),
                  b_dn=(0.02 * rng.standard_normal((E, H))).astype(np.float32))
    what = f"case {case}: {fmt} E={E} H={H} I={I} T={T} k={k} flags={flags:#x} variant={variant}"
    out, out32 = layer.forward(flags, **kw)
    assert_rows_within_tolerance(out32, layer.oracle_out(**kw), what)
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("case", range(8))
def test_random_dgrad(e4b, case):
    rng = np.random.default_rng(3000 + case)
    fmt = ("nf4", "mxfp4")[case % 2]
    E = int(rng.integers(1, 9))
    N, K = 64 * int(rng.integers(1, 17)), 64 * int(rng.integers(1, 21))
    counts = rng.integers(0, 400, E)
    counts[rng.random(E) < 0.25] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((E, N, K))).astype(np.float32))
    g = f32_to_bf16_bits(rng.standard_normal((int(offsets[-1]), N)).astype(np.float32))
    packed, scales = gpu_pack(e4b, fmt, dev_bf16(w))
    out32, out = e4b.e4b_grouped_dgrad(fmt, dev_bf16(g), packed, scales,
                                       torch.from_numpy(offsets).to(DEV), out=True)
    torch.cuda.synchronize()
    op, os_ = (onf4 if fmt == "nf4" else omx).quantize_pack(w)
    ref = omoe.dgrad(fmt, op, os_, g, offsets)
    what = f"case {case}: {fmt} E={E} N={N} K={K} rows={counts.tolist()}"
    if len(ref):
        assert_rows_within_tolerance(host(out32), ref, what)
    assert_out_is_rne_of_f32(host(out), host(out32))


@pytest.mark.parametrize("case", range(8))
def test_random_int4_gemv(e4b, case):
    rng = np.random.default_rng(4000 + case)
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(E, 8) + 1))
    N, K = 16 * int(rng.integers(1, 40)), 128 * int(rng.integers(1, 33))
    T = int(rng.integers(1, 80))
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((E, N, K))).astype(np.float32))
    x = f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    packed, scales = e4b.e4b_pack_int4_b32(dev_bf16(w))
    _, _, off, slots = e4b.e4b_route_permute(torch.from_numpy(logits).to(DEV), k)
    out = e4b.e4b_gemv_int4_b32(packed, scales, dev_bf16(x), k, off, slots)
    torch.cuda.synchronize()
    op, os_ = oi4.quantize_pack(w)
    np.testing.assert_array_equal(host(packed), op)
    ref, mag = oi4.grouped_gemv(op, os_, x, k, host(off), host(slots))
    tol = (K // 32 + 16) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(host(out).astype(np.float64) - ref)
    assert np.all(err <= tol), f"case {case}: E={E} N={N} K={K} T={T} k={k}: worst {np.max(err - tol):.3e}"
