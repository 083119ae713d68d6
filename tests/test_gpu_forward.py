"""GPU MoE forward vs the float64 oracle, to the per-row tolerance
max|gpu - oracle| <= 8e-3 * ||oracle row||_2 / sqrt(H) + 1e-3, applied to the float32 value
the bf16 output is rounded from; the bf16 output must be that value rounded to nearest even."""
import numpy as np
import pytest
import torch

from gpu_helpers import (Layer, assert_out_is_rne_of_f32, assert_rows_within_tolerance,
                         host, random_layer)
from moe_inputs import WORKLOADS, make_logits, make_weights, make_x

pytestmark = pytest.mark.gpu

PATHS = {"auto": 0, "gemm": 1, "gemv": 2}


@pytest.fixture(scope="module")
def tiny(e4b):
    wl = WORKLOADS["tiny_nf4"]
    return Layer(e4b, "nf4", make_x(wl), make_logits(wl), make_weights(wl, "gate_up"),
                 make_weights(wl, "down"), wl.k)


@pytest.mark.parametrize("path", list(PATHS))
def test_tiny_nf4_all_tokens(tiny, path):
    out, out32 = tiny.forward(PATHS[path])
    ref = tiny.oracle_out()
    assert_rows_within_tolerance(out32, ref, f"tiny_nf4/{path}")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("E,H,I,T,k", [
    (8, 256, 512, 64, 2),      # the tiny workload's shape
    (3, 320, 192, 37, 2),      # ragged: I not a multiple of the N tile, T odd
    (5, 128, 64, 300, 5),      # k = E, several M tiles per expert
    (16, 64, 128, 9, 4),       # most experts empty
    (1, 192, 128, 40, 1),      # one expert: a dense SwiGLU MLP
    (2, 128, 128, 700, 2),     # >= 384 rows per expert: 256-row tiles, ragged last tile
])
def test_small_layers(e4b, fmt, path, E, H, I, T, k):
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=E * 7 + T)
    out, out32 = layer.forward(PATHS[path])
    assert_rows_within_tolerance(out32, layer.oracle_out(), f"{fmt}/{path}/{E},{H},{I},{T},{k}")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("T", [1100, 1050])
def test_all_tokens_on_one_expert(e4b, fmt, T):
    """A router biased so that every token picks expert 3 (top-1): one expert holds every row
    (a mean of 69 rows per expert, so 128-row tiles: 8 full tiles and a 76-row last tile at
    T = 1100, 8 and a 26-row tail on the streaming kernel at T = 1050), the other 15 none."""
    bias = np.zeros(16, np.float32)
    bias[3] = 40.0
    layer = random_layer(e4b, fmt, 16, 256, 192, T, 1, seed=T, logit_bias=bias)
    out, out32 = layer.forward(PATHS["auto"])
    assert_rows_within_tolerance(out32, layer.oracle_out(), f"{fmt} one expert T={T}")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_every_expert_for_every_token(e4b, fmt):
    """k = E = 64, the largest top-k the router takes: each token's row goes to all 64 experts."""
    layer = random_layer(e4b, fmt, 64, 128, 64, 20, 64, seed=64)
    out, out32 = layer.forward(PATHS["auto"])
    assert_rows_within_tolerance(out32, layer.oracle_out(), f"{fmt} k=E=64")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.timeout(300)
def test_tails_in_the_last_round(e4b):
    """An expert's short last piece (at most a quarter tile: a tail) runs as one main MFMA tile
    when its GEMM launch fills at least four rounds of the CUs and the last round has free
    slots, else as 16-row tiles on the streaming kernel.  This layer (E=16, H=256, I=3200,
    top-4, T=2048: about 512 rows per expert, 256-row tiles) has several tails; its gate_up
    launch (25 column tiles per row tile) fills four rounds and takes most of them, its down
    launch (one column tile, one round) none, so one forward runs absorbed tails, streamed
    gate_up tails and streamed down tails together."""
    from oracle import route as oroute
    E, H, I, T, k = 16, 256, 3200, 2048, 4
    layer = random_layer(e4b, "nf4", E, H, I, T, k, seed=1)
    counts = np.bincount(oroute.topk(layer.logits, k).ravel(), minlength=E)
    bm, tail = 256, 64
    n_tails = int(sum(1 for c in counts if 0 < c % bm <= tail))
    regular = int(sum(c // bm if 0 < c % bm <= tail else -(-c // bm) for c in counts))
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = regular * (-(-I // 128))
    rounds = -(-wgs // n_cu)
    absorbed = min(n_tails, (rounds * n_cu - wgs) // (-(-I // 128))) if rounds >= 4 else 0
    print(f"tails {n_tails}, gate_up: {rounds} rounds, {absorbed} tails as main tiles")
    assert 0 < absorbed < n_tails, (n_tails, rounds, absorbed)
    out, out32 = layer.forward(PATHS["auto"])
    assert_rows_within_tolerance(out32, layer.oracle_out(), "tails in the last round")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("E,H,I,T,k", [
    (4, 2880, 192, 5, 2),      # gate_up K = 2880: 12 K steps, the last partial; few items, so K is
                               # split over the waves (some take two steps)
    (3, 128, 2112, 7, 1),      # down K = 2112: last step of 64 (K split: wave 0 takes steps 0 and 8)
    (32, 512, 1024, 200, 4),   # more work items than resident workgroups: several items each
])
def test_streaming_path_long_k_and_many_items(e4b, fmt, E, H, I, T, k):
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=H + I + T)
    for path in (PATHS["gemv"], PATHS["gemm"]):
        out, out32 = layer.forward(path)
        assert_rows_within_tolerance(out32, layer.oracle_out(), f"{fmt}/{path}/{E},{H},{I},{T},{k}")
        assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_skewed_routing_with_empty_experts_and_a_hot_expert(e4b, fmt):
    E = 12
    bias = np.full(E, -30.0)
    bias[3] = 10.0                                    # every token picks expert 3 ...
    bias[7] = 5.0                                     # ... and 7; the rest are empty
    layer = random_layer(e4b, fmt, E, 256, 256, 600, 2, seed=5, logit_bias=bias)
    for path in PATHS.values():
        out, out32 = layer.forward(path)
        assert_rows_within_tolerance(out32, layer.oracle_out(), f"{fmt}/skewed/{path}")


def test_paths_agree_and_are_deterministic(tiny):
    a = tiny.forward(1)
    b = tiny.forward(1)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0])
    c = tiny.forward(2)
    d = tiny.forward(2)
    assert np.array_equal(c[1], d[1])


def test_empty_batch(e4b, tiny):
    x = torch.zeros((0, tiny.H), dtype=torch.bfloat16, device="cuda:0")
    lg = torch.zeros((0, tiny.E), dtype=torch.float32, device="cuda:0")
    ids, w, off, slots = e4b.e4b_route_permute(lg, tiny.k)
    out, _ = e4b.e4b_moe_forward("nf4", x, tiny.gp, tiny.gs, tiny.dp, tiny.ds, w, off, slots, tiny.k)
    torch.cuda.synchronize()
    assert out.shape == (0, tiny.H)


def test_zero_input_gives_zero_output(e4b, tiny):
    x = torch.zeros_like(tiny.x)
    ids, w, off, slots = tiny.route()
    out, out32 = e4b.e4b_moe_forward("nf4", x, tiny.gp, tiny.gs, tiny.dp, tiny.ds, w, off, slots,
                                     tiny.k, out_f32=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out32).item() == 0


@pytest.mark.parametrize("path", [1, 2])
def test_graph_replay_matches_eager(e4b, path):
    """route + forward captured in a HIP graph: every replay (with eager work and
    synchronisations in between) reproduces the eager result bit for bit, and that result is
    within the per-row bound of the float64 oracle."""
    layer = random_layer(e4b, "nf4", 16, 256, 256, 24, 4, seed=11)
    T, k, E = layer.T, layer.k, layer.E
    dev = "cuda:0"
    route_out = (torch.empty((T, k), dtype=torch.int32, device=dev),
                 torch.empty((T, k), dtype=torch.float32, device=dev),
                 torch.empty((E + 1,), dtype=torch.int32, device=dev),
                 torch.empty((T * k,), dtype=torch.int32, device=dev))
    rws = torch.empty(max(256, e4b.e4b_route_workspace_bytes(T, E, k)), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(256, e4b.e4b_moe_workspace_bytes("nf4", E, layer.H, layer.I, T, k, path)),
                      dtype=torch.uint8, device=dev)
    out = torch.empty((T, layer.H), dtype=torch.bfloat16, device=dev)
    out32 = torch.empty((T, layer.H), dtype=torch.float32, device=dev)

    def step():
        ids, w, off, slots = e4b.e4b_route_permute(layer.logits_dev, k, ws=rws, out=route_out)
        e4b.e4b_moe_forward("nf4", layer.x, layer.gp, layer.gs, layer.dp, layer.ds, w, off, slots, k,
                            out=out, out_f32=out32, ws=fws, path=path)

    step()
    torch.cuda.synchronize()
    ref = out32.clone()
    assert_rows_within_tolerance(host(ref), layer.oracle_out(), f"graph/{path}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out32.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out32, ref)
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out32, ref)


# ------------------------------------------------- clamped-GLU / interleaved / bias variant

VARIANT_CASES = [
    # fmt, flags (path | tile), E, H, I, T, k
    ("mxfp4", 0x0, 8, 256, 256, 300, 2),    # automatic: 128-row tiles, tail tiles
    ("nf4", 0xC, 2, 256, 256, 270, 2),      # 256-row tiles + streaming tail tiles (slot order)
    ("mxfp4", 0xC, 2, 256, 320, 270, 2),    # the same in MXFP4 (natural order tails)
    ("nf4", 0x4, 4, 256, 256, 64, 2),       # 32-row tiles
    ("nf4", 0x8, 2, 256, 256, 300, 2),      # 128-row tiles: full tiles (buffer-store epilogue) + a partial one
    ("mxfp4", 0x8, 2, 256, 320, 300, 2),    # the same in MXFP4
    ("mxfp4", 0x2, 16, 256, 256, 16, 4),    # streaming path
    ("nf4", 0x0, 16, 512, 256, 8, 4),       # automatic: streaming path
]


@pytest.mark.parametrize("fmt,flags,E,H,I,T,k", VARIANT_CASES)
def test_clamped_glu_interleaved_with_biases(e4b, fmt, flags, E, H, I, T, k):
    layer = random_layer(e4b, fmt, E, H, I, T, k, seed=E * 7 + T + (flags << 4))
    rng = np.random.default_rng(T + E)
    # biases wide enough that some gate values pass the clamp at 7 and some up values leave [-7, 7]
    b_gu = (4.0 * rng.standard_normal((E, 2 * I))).astype(np.float32)
    b_dn = rng.standard_normal((E, H)).astype(np.float32)
    for interleaved in (True, False):
        out, out32 = layer.forward(flags, act="clamped_glu", interleaved=interleaved, b_gu=b_gu, b_dn=b_dn)
        ref = layer.oracle_out(act="clamped_glu", interleaved=interleaved, b_gu=b_gu, b_dn=b_dn)
        assert_rows_within_tolerance(out32, ref, f"{fmt} flags={flags:#x} interleaved={interleaved}")
        assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("flags", [0x0, 0x2, 0x8])
def test_swiglu_with_one_bias_and_interleaved_rows(e4b, flags):
    # 0x8: two experts of ~400 rows on 128-row tiles, so most tiles are full
    E, H, I, T, k = 2 if flags == 0x8 else 8, 256, 256, 48 if flags == 0x2 else 400, 2
    layer = random_layer(e4b, "nf4", E, H, I, T, k, seed=31 + flags)
    rng = np.random.default_rng(5)
    b_gu = rng.standard_normal((E, 2 * I)).astype(np.float32)
    b_dn = rng.standard_normal((E, H)).astype(np.float32)
    for kw in (dict(b_gu=b_gu), dict(b_dn=b_dn), dict(interleaved=True, b_gu=b_gu)):
        out, out32 = layer.forward(flags, **kw)
        assert_rows_within_tolerance(out32, layer.oracle_out(**kw), f"flags={flags:#x} {sorted(kw)}")


def test_binding_rejects_mismatched_tensors(e4b, tiny):
    """Every tensor of e4b_moe_forward is checked against the shape fmt, E, H, I, T and k
    imply before the library is called (no launch on inconsistent buffers)."""
    ids, w, off, slots = tiny.route()
    torch.cuda.synchronize()
    args = dict(fmt="nf4", x=tiny.x, w_gu=tiny.gp, s_gu=tiny.gs, w_dn=tiny.dp, s_dn=tiny.ds,
                topk_w=w, expert_offsets=off, sorted_slots=slots, k=tiny.k)

    def bad(**kw):
        a = dict(args, **kw)
        with pytest.raises((ValueError, TypeError)):
            e4b.e4b_moe_forward(a.pop("fmt"), a.pop("x"), a.pop("w_gu"), a.pop("s_gu"), a.pop("w_dn"),
                                a.pop("s_dn"), a.pop("topk_w"), a.pop("expert_offsets"),
                                a.pop("sorted_slots"), a.pop("k"), **a)

    bad(fmt="mxfp4")                                   # NF4 stacks read as MXFP4
    bad(expert_offsets=off[:-1].contiguous())          # one expert too few
    bad(w_gu=tiny.gp[:, : tiny.gp.shape[1] // 2].contiguous())   # half the gate_up rows
    bad(s_dn=tiny.ds.to(torch.float16))                # wrong scale dtype
    bad(topk_w=w[:, :1].contiguous())                  # k = 1 weights for k = 2
    bad(sorted_slots=slots[:-1].contiguous())
    bad(x=tiny.x.t())                                  # not contiguous
    bad(out=torch.empty((tiny.T, tiny.H + 64), dtype=torch.bfloat16, device="cuda:0"))
    bad(out_f32=torch.empty((tiny.T, tiny.H), dtype=torch.float16, device="cuda:0"))
    bad(w_dn=tiny.dp.cpu())                            # host tensor
    out, _ = e4b.e4b_moe_forward(**{**args, "fmt": "nf4"})
    torch.cuda.synchronize()
    assert out.shape == (tiny.T, tiny.H)
