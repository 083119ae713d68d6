"""The atomic weighted scatter-combine (E4B_COMBINE_ATOMIC) against the float64 oracle.

With the flag the down GEMM adds topk_w * y straight into a float32 [T, H] accumulator with
atomic adds (the combine of the grouped-nf4-gemm 0.25.0 glue kernels, project description
opening section, fused into the down GEMM's epilogue); the summation order of a token's k
contributions is then not fixed, so the checks are the same per-row bound against the oracle
as for the default combine, never bit equality between calls."""
import numpy as np
import pytest
import torch

from gpu_helpers import (assert_out_is_rne_of_f32, assert_rows_within_tolerance, host,
                         random_layer)
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

ATOMIC = 0x100


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("flags,E,H,I,T,k", [
    (0x0, 8, 256, 512, 64, 2),      # automatic: MFMA tiles (a mean of 16 rows per expert)
    (0x0, 3, 320, 192, 37, 2),      # ragged column tile, odd T
    (0x0, 5, 128, 64, 300, 5),      # k = E: every token's rows in every expert
    (0x1, 16, 64, 128, 9, 4),       # MFMA path forced, most experts empty
    (0xC, 2, 256, 256, 270, 2),     # 256-row tiles + 16-row tail tiles on the streaming kernel
    (0x8, 8, 256, 256, 300, 2),     # 128-row tiles + tails
    (0x4, 4, 256, 256, 64, 2),      # 32-row tiles
    (0x2, 16, 256, 256, 16, 4),     # streaming path: the flag leaves the ordered combine
])
def test_atomic_combine_small_layers(e4b, fmt, flags, E, H, I, T, k):
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=E * 11 + T)
    ref = layer.oracle_out()
    out, out32 = layer.forward(flags | ATOMIC)
    assert_rows_within_tolerance(out32, ref, f"{fmt} flags={flags:#x} atomic")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt,flags,E,H,I,T,k", [
    ("mxfp4", 0x0, 8, 256, 256, 300, 2),
    ("nf4", 0xC, 2, 256, 256, 270, 2),
])
def test_atomic_combine_with_biases(e4b, fmt, flags, E, H, I, T, k):
    """Down bias added before the routing weight: out += w * (h . W + b)."""
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=3 * T + E)
    rng = np.random.default_rng(T)
    b_gu = (4.0 * rng.standard_normal((E, 2 * I))).astype(np.float32)
    b_dn = rng.standard_normal((E, H)).astype(np.float32)
    out, out32 = layer.forward(flags | ATOMIC, act="clamped_glu", interleaved=True, b_gu=b_gu, b_dn=b_dn)
    ref = layer.oracle_out(act="clamped_glu", interleaved=True, b_gu=b_gu, b_dn=b_dn)
    assert_rows_within_tolerance(out32, ref, f"{fmt} atomic with biases")
    assert_out_is_rne_of_f32(out, out32)


def test_atomic_combine_without_out_f32(e4b):
    """No out_f32: the accumulator lives in the workspace; the bf16 output is still within the
    bound plus its own rounding (half an ulp of bf16, 2^-9 relative)."""
    layer = random_layer(e4b, "nf4", 6, 256, 192, 500, 3, seed=5)
    ids, w, off, slots = layer.route()
    out, out32 = layer.e4b.e4b_moe_forward("nf4", layer.x, layer.gp, layer.gs, layer.dp, layer.ds, w, off,
                                           slots, layer.k, out_f32=None, path=ATOMIC)
    torch.cuda.synchronize()
    assert out32 is None
    ref = layer.oracle_out()
    got = (host(out).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tau = omoe.tolerance(ref)[:, None] + np.abs(ref) * 2.0 ** -8
    assert np.all(np.abs(got - ref) <= tau)


def test_atomic_combine_repeated_calls_and_graph(e4b):
    """Calls in a row (the accumulator is cleared by each call) and graph replays, each checked
    against the oracle: a stale accumulator would double the output."""
    E, H, I, T, k = 8, 256, 256, 400, 2
    layer = random_layer(e4b, "nf4", E, H, I, T, k, seed=9)
    ref = layer.oracle_out()
    dev = layer.x.device
    route_out = (torch.empty((T, k), dtype=torch.int32, device=dev),
                 torch.empty((T, k), dtype=torch.float32, device=dev),
                 torch.empty((E + 1,), dtype=torch.int32, device=dev),
                 torch.empty((T * k,), dtype=torch.int32, device=dev))
    rws = torch.empty(max(256, e4b.e4b_route_workspace_bytes(T, E, k)), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(256, e4b.e4b_moe_workspace_bytes("nf4", E, H, I, T, k, ATOMIC)),
                      dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    out32 = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step():
        ids, w, off, slots = e4b.e4b_route_permute(layer.logits_dev, k, ws=rws, out=route_out)
        e4b.e4b_moe_forward("nf4", layer.x, layer.gp, layer.gs, layer.dp, layer.ds, w, off, slots, k,
                            out=out, out_f32=out32, ws=fws, path=ATOMIC)

    for i in range(3):
        step()
        torch.cuda.synchronize()
        assert_rows_within_tolerance(host(out32), ref, f"eager call {i}")
        assert_out_is_rne_of_f32(host(out), host(out32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out32.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_rows_within_tolerance(host(out32), ref, f"graph replay {i}")
        assert_out_is_rne_of_f32(host(out), host(out32))
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("case", range(6))
def test_atomic_combine_random_shapes(e4b, case):
    """Seeded random shapes (as in the random-shape forward tests) with the atomic combine on the
    MFMA tile path, every row-tile size."""
    rng = np.random.default_rng(5000 + case)
    fmt = ("nf4", "mxfp4")[case % 2]
    E = int(rng.integers(1, 25))
    k = int(rng.integers(1, min(E, 8) + 1))
    H, I = 64 * int(rng.integers(1, 17)), 64 * int(rng.integers(1, 13))
    T = int(rng.integers(1, 600))
    flags = 0x1 | (0x0, 0x4, 0x8, 0xC)[case % 4]
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=6000 + case)
    out, out32 = layer.forward(flags | ATOMIC)
    what = f"case {case}: {fmt} E={E} H={H} I={I} T={T} k={k} flags={flags:#x}"
    assert_rows_within_tolerance(out32, layer.oracle_out(), what)
    assert_out_is_rne_of_f32(out, out32)
