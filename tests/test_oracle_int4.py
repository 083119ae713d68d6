"""Pins for the int4-b32 part of the oracle (oracle/int4.py): each checks it against something
other than itself — exact grids, brute-force nearest codes, hand-made bytes, pure-Python
integer loops, and the float64 product of the separately decoded weight and activation."""
import numpy as np
import pytest

from moe_inputs import f32_to_bf16_bits
from oracle import int4


def test_grid_weights_round_trip_exactly():
    """Weights s*q with s a power of two and a +-7 in every block: the packer must return s and
    q unchanged, and decoding must give the weights back exactly."""
    rng = np.random.default_rng(0)
    N, K = 16, 128
    q = rng.integers(-8, 8, (N, K))
    q[:, ::32] = np.where(rng.random((N, K // 32)) < 0.5, 7, -7)
    q = np.maximum(q, -7)                  # a -8 would make absmax 8s
    s = 2.0 ** -6
    w = (q * s).astype(np.float32)
    packed, scales = int4.quantize_pack(w)
    assert packed.shape == (N, K // 2) and scales.shape == (N, K // 32)
    assert np.all(scales.view(np.float16).astype(np.float64) == s)
    np.testing.assert_array_equal(int4.unpack_codes(packed), q.astype(np.int8))
    np.testing.assert_array_equal(int4.dequantize(packed, scales), w.astype(np.float64))


def test_nibble_order_and_twos_complement():
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1], w[0, 2], w[0, 3] = 1.0, -1.0, 7.0, -7.0
    packed, scales = int4.quantize_pack(w)
    assert scales.view(np.float16)[0, 0] == np.float16(1.0)
    assert packed[0, 0] == 0xF1          # element 0 (q = 1) low nibble, element 1 (q = -1) high
    assert packed[0, 1] == 0x97          # q = 7 low, q = -7 (0b1001) high
    assert np.all(packed[0, 2:] == 0)


def test_codes_are_the_nearest_level_of_the_stored_scale():
    """Brute force over the 16 levels s*q: the code is the nearest one, an exact tie goes to
    the even q (round half to even), and values past the range saturate."""
    rng = np.random.default_rng(1)
    w = (0.02 * rng.standard_normal((8, 256))).astype(np.float32)
    packed, scales = int4.quantize_pack(w)
    q = int4.unpack_codes(packed).astype(np.int64)
    s = np.repeat(scales.view(np.float16).astype(np.float32), 32, axis=-1)
    levels = np.arange(-8, 8)
    for n in range(8):
        for k in range(256):
            r = np.float32(w[n, k]) / s[n, k]           # the float32 quotient the rule rounds
            d = np.abs(float(r) - levels)
            best = levels[d == d.min()]
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[n, k] == want, (n, k)


def test_scale_is_absmax_over_7_in_fp16_and_the_max_maps_to_7():
    rng = np.random.default_rng(2)
    w = (0.03 * rng.standard_normal((4, 96))).astype(np.float32)
    packed, scales = int4.quantize_pack(w)
    a = np.abs(w.reshape(4, 3, 32)).max(-1)
    np.testing.assert_array_equal(scales.view(np.float16), (a / np.float32(7)).astype(np.float16))
    q = int4.unpack_codes(packed).reshape(4, 3, 32).astype(np.int64)
    assert np.all(np.abs(q).max(-1) == 7)


def test_zero_block_and_bf16_input():
    w = np.zeros((2, 64), np.float32)
    w[1, 40] = 0.5
    packed, scales = int4.quantize_pack(f32_to_bf16_bits(w))
    assert np.all(scales[0] == 0) and scales[1, 0] == 0 and np.all(packed[0] == 0)
    assert int4.unpack_codes(packed)[1, 40] == 7


def test_size_is_4_5_bits_per_weight():
    assert int4.bytes_per_element() == 0.5625
    packed, scales = int4.quantize_pack(np.ones((8, 256), np.float32))
    assert packed.nbytes + scales.nbytes == 8 * 256 * 0.5625


def test_activation_quantiser_on_exact_grid_and_ties():
    """x = s_x * m with s_x = absmax / 127 exactly representable: the codes are m; a value at
    an exact half step rounds to the even code."""
    sx = np.float32(127.0 / 127.0)
    m = np.array([127, -127, 3, 0, -64, 5], np.float32)
    q, s = int4.quantize_act(m[None, :] * sx)
    assert s[0] == np.float32(1.0)
    np.testing.assert_array_equal(q[0], m.astype(np.int8))
    x = np.array([[127.0, 2.5, -2.5, 3.5, -0.5, 0.5]], np.float32)
    q, s = int4.quantize_act(x)
    np.testing.assert_array_equal(q[0], np.array([127, 2, -2, 4, 0, 0], np.int8))
    q, s = int4.quantize_act(np.zeros((1, 8), np.float32))
    assert s[0] == 0 and np.all(q == 0)


def test_block_sums_match_pure_python_loops():
    rng = np.random.default_rng(3)
    codes = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    qx = rng.integers(-127, 128, 64).astype(np.int8)
    I = int4.block_sums(codes, qx)
    for n in range(5):
        for b in range(2):
            ref = sum(int(codes[n, k]) * int(qx[k]) for k in range(32 * b, 32 * b + 32))
            assert I[n, b] == ref


def test_gemv_equals_decoded_weight_times_decoded_activation():
    """The integer form against an independent float64 product of the separately decoded
    weight (s*q) and activation (s_x*q_x)."""
    rng = np.random.default_rng(4)
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((48, 256))).astype(np.float32))
    x = f32_to_bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    packed, scales = int4.quantize_pack(w)
    qx, sx = int4.quantize_act(x)
    W = int4.dequantize(packed, scales)
    for t in range(3):
        y, mag = int4.gemv_rows(packed, scales, qx[t], sx[t])
        ref = W @ (qx[t].astype(np.float64) * float(sx[t]))
        np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * float(np.max(mag)))
        assert np.all(mag >= np.abs(y))


def test_grouped_gemv_follows_the_routing():
    """Sorted row p of expert e takes token slots[p] // k through expert e; a dense layer is
    the one-expert case with every token routed to it."""
    rng = np.random.default_rng(5)
    E, N, K, T, k = 3, 16, 64, 4, 2
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((E, N, K))).astype(np.float32))
    x = f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    packed, scales = int4.quantize_pack(w)
    ids = np.array([[0, 2], [2, 1], [0, 1], [2, 0]])
    slots = np.argsort(ids.reshape(-1), kind="stable")
    counts = np.bincount(ids.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    y, _ = int4.grouped_gemv(packed, scales, x, k, offsets, slots)
    qx, sx = int4.quantize_act(x)
    for p, s in enumerate(slots):
        t, e = s // k, ids.reshape(-1)[s]
        ref, _ = int4.gemv_rows(packed[e], scales[e], qx[t], sx[t])
        np.testing.assert_array_equal(y[p], ref)
    yd, _ = int4.grouped_gemv(packed[:1], scales[:1], x, 1, [0, T], np.arange(T))
    W = int4.dequantize(packed[0], scales[0])
    ref = (qx.astype(np.float64) * sx[:, None].astype(np.float64)) @ W.T
    np.testing.assert_allclose(yd, ref, rtol=1e-12, atol=1e-12)
