"""The MXFP4 gate_up on gfx950's block-scaled fp8 x fp4 instruction (flag E4B_MXFP4_SCALED): the
released e2m1 bytes and e8m0 scales go to the matrix unit as they are and the bf16 activations as
exact fp8 hi + lo parts.  Checked against the float64 oracle to the per-row tolerance (fp32
output) with the bf16 output its round to nearest even: small and ragged layers on both row
tiles (with the tail tiles of the streaming kernel), the expert variant (interleaved rows,
biases, clamped GLU), the operand-range edges with a purely relative bound, and the full-size
MXFP4 layer with every token, where it must also beat the dequantise-to-bf16 comparator."""
import numpy as np
import pytest
import torch

import fullsize_oracle as fo
from gpu_helpers import (Layer, assert_out_is_rne_of_f32, assert_rows_within_tolerance, host,
                         random_layer)
from moe_inputs import WORKLOADS, f32_to_bf16_bits, make_bias, make_expert_weight, make_logits, make_x

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCALED = 0x40
GEMM, T128, T256 = 0x1, 0x8, 0xC


@pytest.mark.parametrize("tile", [T128, T256], ids=["tile128", "tile256"])
@pytest.mark.parametrize("E,H,I,T,k", [
    (8, 256, 512, 64, 2),
    (3, 320, 192, 37, 2),      # ragged: I not a multiple of the N tile, K of 5 steps
    (5, 128, 64, 300, 5),      # several tiles per expert
    (16, 64, 128, 9, 4),       # most experts empty, one K step
    (2, 128, 128, 700, 2),     # 256-row tiles with a ragged last tile and tails
    (4, 2880, 256, 300, 2),    # K = 2880: 45 steps, no padding
])
def test_scaled_route_small_layers(e4b, tile, E, H, I, T, k):
    lay = random_layer(e4b, "mxfp4", E, H, I, T, k, seed=E * 7 + T)
    out, out32 = lay.forward(path=GEMM | tile | SCALED)
    assert_rows_within_tolerance(out32, lay.oracle_out(), f"scaled E{E} H{H} I{I} T{T}")
    assert_out_is_rne_of_f32(out, out32)


def test_scaled_route_expert_variant(e4b):
    lay = random_layer(e4b, "mxfp4", 8, 256, 256, 200, 2, seed=41)
    rng = np.random.default_rng(42)
    b_gu = (0.02 * rng.standard_normal((8, 512))).astype(np.float32)
    b_dn = (0.02 * rng.standard_normal((8, 256))).astype(np.float32)
    out, out32 = lay.forward(path=GEMM | T128 | SCALED, act="clamped_glu", interleaved=True, b_gu=b_gu, b_dn=b_dn)
    ref = lay.oracle_out(act="clamped_glu", interleaved=True, b_gu=b_gu, b_dn=b_dn)
    assert_rows_within_tolerance(out32, ref, "scaled variant")
    assert_out_is_rne_of_f32(out, out32)


@pytest.mark.parametrize("name,xs,ws,big", [
    ("x_near_fp16_max", 1.0, 2.0 ** -6, 65280.0),
    ("weights_x2^8", 2.0 ** -4, 2.0 ** 8, None),
    ("weights_x2^-12", 2.0 ** 12, 2.0 ** -12, None),
    ("x_tiny_elements", 1.0, 1.0, None),
])
def test_scaled_route_range_edges(e4b, name, xs, ws, big):
    """Relative bound per row (no absolute term).  x_tiny_elements puts elements 2^-12 below
    their block's largest in every block: the part of the activation split that rounds."""
    E, H, I, T, K_TOP = 4, 256, 256, 256, 2
    rng = np.random.default_rng(17)
    x = rng.standard_normal((T, H)).astype(np.float32) * np.float32(xs)
    if big is not None:
        cols = rng.integers(0, H, size=(T, 2))
        x[np.arange(T)[:, None], cols] = np.where(rng.random((T, 2)) < 0.5, -1.0, 1.0).astype(np.float32) * np.float32(big)
    if name == "x_tiny_elements":
        x[:, 1::4] *= np.float32(2.0 ** -12)
    gu = (0.02 * rng.standard_normal((E, 2 * I, H))).astype(np.float32) * np.float32(ws)
    dn = (0.02 * rng.standard_normal((E, H, I))).astype(np.float32) * np.float32(ws)
    lg = rng.standard_normal((T, E), dtype=np.float32)
    lay = Layer(e4b, "mxfp4", f32_to_bf16_bits(x), lg, f32_to_bf16_bits(gu), f32_to_bf16_bits(dn), K_TOP)
    _, got = lay.forward(path=GEMM | T128 | SCALED)
    ref = lay.oracle_out()
    assert np.all(np.isfinite(got))
    bound = 8e-3 * np.linalg.norm(ref, axis=1) / np.sqrt(H)
    ratio = np.max(np.abs(got.astype(np.float64) - ref), axis=1) / bound
    print(f"scaled {name}: worst relative err/bound {ratio.max():.3f}")
    assert np.all(ratio <= 1.0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", [False, True], ids=["swiglu", "clamped_glu"])
def test_scaled_route_full_size_mxfp4_layer(e4b, variant):
    wl = WORKLOADS["mxfp4_moe"]
    packed = {}
    for which, (N, K) in (("gate_up", (2 * wl.I, wl.H)), ("down", (wl.H, wl.I))):
        w = torch.empty((wl.E, N, K), dtype=torch.bfloat16, device=DEV)
        for e in range(wl.E):
            w[e].copy_(torch.from_numpy(make_expert_weight(wl, which, e).view(np.int16)).view(torch.bfloat16))
        packed[which] = e4b.e4b_pack_mxfp4(w)
        del w
    x = torch.from_numpy(make_x(wl).view(np.int16)).to(DEV).view(torch.bfloat16)
    logits = torch.from_numpy(make_logits(wl)).to(DEV)
    ids, w, off, slots = e4b.e4b_route_permute(logits, wl.k)
    kw = {}
    if variant:
        kw = dict(act="clamped_glu", interleaved=True, b_gu=torch.from_numpy(make_bias(wl, "gate_up")).to(DEV),
                  b_dn=torch.from_numpy(make_bias(wl, "down")).to(DEV))
    (gp, gs), (dp, ds) = packed["gate_up"], packed["down"]
    out, out32 = e4b.e4b_moe_forward("mxfp4", x, gp, gs, dp, ds, w, off, slots, wl.k, out_f32=True,
                                     path=SCALED, **kw)
    torch.cuda.synchronize()
    r_ids, r_w, _, r_off, r_slots = fo.routed(wl)
    np.testing.assert_array_equal(host(slots), r_slots)
    ref, cmp_ = fo.expected(wl, np.arange(wl.T), r_ids, r_w, variant)
    o32 = host(out32)
    worst = assert_rows_within_tolerance(o32, ref, "scaled full size")
    assert_out_is_rne_of_f32(host(out), o32)
    e_f, e_c = o32.astype(np.float64) - ref, cmp_ - ref
    print(f"scaled full size ({'variant' if variant else 'swiglu'}): worst err/tol {worst:.3f}; RMS error "
          f"{np.sqrt(np.mean(e_f ** 2)):.3e} vs dequant-bf16 {np.sqrt(np.mean(e_c ** 2)):.3e}")
    assert np.sqrt(np.mean(e_f ** 2)) < np.sqrt(np.mean(e_c ** 2)) and np.abs(e_f).max() < np.abs(e_c).max()
