"""The forward at the edges of the operand ranges stated in include/e4b.h ("Operand ranges"):
activations near fp16's largest value, and weights scaled by 2^8 and 2^-12 (NF4 absmax near
13 and near 2^-16; MXFP4 scale exponents near 2 and -18), with the activations rescaled so the
intermediate h stays in range.  Each is checked against the float64 oracle with a purely
relative bound per row, max |gpu - oracle| <= 8e-3 * ||oracle row||_2 / sqrt(H), so the 1e-3
absolute term of the usual bound cannot hide an error at small scales."""
import numpy as np
import pytest

from gpu_helpers import Layer
from moe_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

E, H, I, T, K_TOP = 4, 256, 256, 256, 2


def _layer(e4b, fmt, seed, x_scale, w_scale, big_x=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32) * np.float32(x_scale)
    if big_x is not None:        # two elements of every token near fp16's largest value
        cols = rng.integers(0, H, size=(T, 2))
        sign = np.where(rng.random((T, 2)) < 0.5, -1.0, 1.0).astype(np.float32)
        x[np.arange(T)[:, None], cols] = sign * np.float32(big_x)
    gu = (0.02 * rng.standard_normal((E, 2 * I, H))).astype(np.float32) * np.float32(w_scale)
    dn = (0.02 * rng.standard_normal((E, H, I))).astype(np.float32) * np.float32(w_scale)
    lg = rng.standard_normal((T, E), dtype=np.float32)
    return Layer(e4b, fmt, f32_to_bf16_bits(x), lg, f32_to_bf16_bits(gu), f32_to_bf16_bits(dn), K_TOP)


CASES = [
    # name, activation scale, weight scale, large activation value
    ("x_near_fp16_max", 1.0, 2.0 ** -6, 65280.0),    # 65280 = largest bf16 below 65504
    ("weights_x2^8", 2.0 ** -4, 2.0 ** 8, None),
    ("weights_x2^-12", 2.0 ** 12, 2.0 ** -12, None),
]


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("path", [1, 2], ids=["gemm", "gemv"])
@pytest.mark.parametrize("name,xs,ws,big", CASES, ids=[c[0] for c in CASES])
def test_forward_at_range_edges(e4b, fmt, path, name, xs, ws, big):
    lay = _layer(e4b, fmt, 17, xs, ws, big)
    _, got = lay.forward(path=path)
    ref = lay.oracle_out()
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    bound = 8e-3 * np.linalg.norm(ref, axis=1) / np.sqrt(H)
    err = np.max(np.abs(got.astype(np.float64) - ref), axis=1)
    ratio = err / bound
    w = int(np.argmax(ratio))
    print(f"{fmt} {name}: worst relative err/bound {ratio[w]:.3f} (row {w}, |row| {np.linalg.norm(ref[w]):.3e})")
    assert np.all(ratio <= 1.0), f"{name}: row {w} err {err[w]:.3e} > {bound[w]:.3e}"
