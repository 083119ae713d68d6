"""The single-launch decode step e4b_moe_decode_step against the float64 oracle: routing
bit-identical to the oracle's and to e4b_route_permute, the fp32 output within the per-row
tolerance, the bf16 output its round to nearest even; on small layers of both formats (ragged
K steps, several expert counts, the expert variant, routing without renormalisation) and on the
128-expert decode layer at T = 1 and 4 with every token checked.  Also: run-to-run identity, the
grid barrier's give-up path forced from the host (tiny spin limit, the kernel still ends and
reports it), and replays of the step from a HIP graph against the eager result."""
import numpy as np
import pytest
import torch

import fullsize_oracle as fo
from gpu_helpers import (assert_out_is_rne_of_f32, assert_rows_within_tolerance, host,
                         random_layer)
from moe_inputs import WORKLOADS, make_expert_weight, make_logits, make_x
from oracle import route as oroute

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def step(e4b, lay, renormalize=True, **kw):
    out, out32, route = e4b.e4b_moe_decode_step(lay.fmt, lay.logits_dev, lay.x, lay.gp, lay.gs, lay.dp,
                                                lay.ds, lay.k, renormalize=renormalize, out_f32=True,
                                                route_out=True, **kw)
    torch.cuda.synchronize()
    return host(out), host(out32), tuple(host(t) for t in route)


def check_routing(e4b, lay, route, renormalize=True):
    ids, w, counts, off, slots = oroute.route(lay.logits, lay.k, renormalize)
    np.testing.assert_array_equal(route[0], ids)
    np.testing.assert_allclose(route[1], w, rtol=2e-6, atol=1e-7)
    np.testing.assert_array_equal(route[2], off)
    np.testing.assert_array_equal(route[3], slots)
    ref = [host(t) for t in lay.route(renormalize)]
    torch.cuda.synchronize()
    for a, b in zip(route, ref):       # bit-identical to the router
        assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


SHAPES = [
    ("nf4", 8, 256, 512, 4, 2),
    ("mxfp4", 16, 320, 192, 8, 4),     # K steps of 256 with a ragged last one (H and I)
    ("nf4", 128, 128, 64, 8, 8),       # 64 routed slots, E > 64
    ("mxfp4", 300, 256, 128, 3, 7),    # E > 256
    ("nf4", 1, 128, 128, 1, 1),        # one expert, one token: a dense SwiGLU MLP
    ("nf4", 64, 256, 256, 1, 64),      # k = E = 64
]


@pytest.mark.parametrize("fmt,E,H,I,T,k", SHAPES, ids=[f"{s[0]}-E{s[1]}-H{s[2]}-I{s[3]}-T{s[4]}-k{s[5]}" for s in SHAPES])
def test_decode_step_small_layers(e4b, fmt, E, H, I, T, k):
    lay = random_layer(e4b, fmt, E, H, I, T, k, seed=E + T)
    out, out32, route = step(e4b, lay)
    check_routing(e4b, lay, route)
    assert_rows_within_tolerance(out32, lay.oracle_out(), f"decode step {fmt}")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_decode_step_expert_variant_and_unnormalised_routing(e4b, fmt):
    lay = random_layer(e4b, fmt, 8, 256, 256, 4, 2, seed=31)
    rng = np.random.default_rng(32)
    b_gu = (0.02 * rng.standard_normal((8, 512))).astype(np.float32)
    b_dn = (0.02 * rng.standard_normal((8, 256))).astype(np.float32)
    dev = lambda b: torch.from_numpy(b).to(DEV)
    out, out32, route = step(e4b, lay, renormalize=False, act="clamped_glu", interleaved=True,
                             b_gu=dev(b_gu), b_dn=dev(b_dn))
    check_routing(e4b, lay, route, renormalize=False)
    from oracle import moe as omoe
    from gpu_helpers import oracle_pack
    gp, gs = oracle_pack(fmt, lay.gu_bits)
    dp, ds = oracle_pack(fmt, lay.dn_bits)
    ids, w, *_ = oroute.route(lay.logits, lay.k, False)
    ref = omoe.forward(fmt, lay.x_bits, gp, gs, dp, ds, ids, w, act="clamped_glu", interleaved=True,
                       b_gu=b_gu.astype(np.float64), b_dn=b_dn.astype(np.float64))
    assert_rows_within_tolerance(out32, ref, f"decode step variant {fmt}")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T", [1, 4])
def test_decode_step_full_size_decode_layer(e4b, T):
    wl = WORKLOADS["finegrained_nf4_decode"].with_T(T)
    packed = {}
    for which, (N, K) in (("gate_up", (2 * wl.I, wl.H)), ("down", (wl.H, wl.I))):
        w = torch.empty((wl.E, N, K), dtype=torch.bfloat16, device=DEV)
        for e in range(wl.E):
            w[e].copy_(torch.from_numpy(make_expert_weight(wl, which, e).view(np.int16)).view(torch.bfloat16))
        packed[which] = e4b.e4b_pack_nf4(w)
        del w
    x = torch.from_numpy(make_x(wl).view(np.int16)).to(DEV).view(torch.bfloat16)
    logits = torch.from_numpy(make_logits(wl)).to(DEV)
    (gp, gs), (dp, ds) = packed["gate_up"], packed["down"]
    out, out32, route = e4b.e4b_moe_decode_step("nf4", logits, x, gp, gs, dp, ds, wl.k, out_f32=True,
                                                route_out=True)
    torch.cuda.synchronize()
    r_ids, r_w, _, r_off, r_slots = fo.routed(wl)
    np.testing.assert_array_equal(host(route[0]), r_ids)
    np.testing.assert_array_equal(host(route[2]), r_off)
    np.testing.assert_array_equal(host(route[3]), r_slots)
    ref, _ = fo.expected(wl, np.arange(T), r_ids, r_w, False)
    worst = assert_rows_within_tolerance(host(out32), ref, f"decode step T={T}")
    assert_out_is_rne_of_f32(host(out), host(out32))
    print(f"decode step T={T}: worst err/tol {worst:.3f}")


def test_decode_step_is_deterministic_and_reuses_its_workspace(e4b):
    lay = random_layer(e4b, "nf4", 128, 256, 128, 4, 8, seed=5)
    ws = torch.zeros(e4b.e4b_decode_workspace_bytes("nf4", 128, 256, 128, 4, 8), dtype=torch.uint8, device=DEV)
    a = step(e4b, lay, ws=ws)
    b = step(e4b, lay, ws=ws)
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[0], b[0])


def test_decode_step_barrier_give_up_is_reported_and_recovers(e4b):
    """A spin limit that gives up at once: the kernel still runs to the end and reports it; the
    next call on the same workspace is correct again."""
    lay = random_layer(e4b, "nf4", 16, 256, 256, 2, 4, seed=8)
    ws = torch.zeros(e4b.e4b_decode_workspace_bytes("nf4", 16, 256, 256, 2, 4), dtype=torch.uint8, device=DEV)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    step(e4b, lay, ws=ws, status=status, spin_limit=-1)
    assert int(status.item()) == 1
    status.fill_(-1)
    out, out32, _ = step(e4b, lay, ws=ws, status=status)
    assert int(status.item()) == 0
    assert_rows_within_tolerance(out32, lay.oracle_out(), "after a give-up")


def test_decode_step_graph_replay_matches_eager(e4b):
    lay = random_layer(e4b, "nf4", 64, 512, 256, 2, 8, seed=12)
    T, H = lay.T, lay.H
    ws = torch.zeros(e4b.e4b_decode_workspace_bytes("nf4", 64, H, 256, T, 8), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    out32 = torch.empty((T, H), dtype=torch.float32, device=DEV)
    run = lambda: e4b.e4b_moe_decode_step("nf4", lay.logits_dev, lay.x, lay.gp, lay.gs, lay.dp, lay.ds, 8,
                                          out=out, out_f32=out32, ws=ws)
    run()
    torch.cuda.synchronize()
    eager = host(out32).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        out32.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out32).view(np.uint32), eager.view(np.uint32)), f"replay {i}"
        x2 = torch.randn(1000, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()


def test_decode_step_rejects_bad_sizes(e4b):
    lay = random_layer(e4b, "nf4", 8, 128, 128, 9, 2, seed=3)
    with pytest.raises(e4b.E4BError):           # T = 9 > 8
        e4b.e4b_moe_decode_step("nf4", lay.logits_dev, lay.x, lay.gp, lay.gs, lay.dp, lay.ds, 2)
