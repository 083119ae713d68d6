"""GPU int4-b32 path vs the oracle (oracle/int4.py): packed bytes, scales and int8 activations
bit-exact; GEMV outputs within the float32 rounding bound of their block sums,
|gpu - oracle| <= (K/32 + 16) * 2^-24 * s_x * sum_b |s * I_b| (each block term is an exact
integer times a scale; only the float32 sums round)."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, dev_bf16, host
from moe_inputs import INT4_WORKLOADS, f32_to_bf16_bits, make_expert_weight, make_logits, make_x
from oracle import int4 as oi4
from oracle import route as oroute

pytestmark = pytest.mark.gpu


def _bits16(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def _assert_gemv_close(got, ref, mag, K, what):
    tol = (K // 32 + 16) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"{what}: at {worst} err {err[worst]:.3e} > tol {tol[worst]:.3e}")


@pytest.mark.parametrize("E,N,K", [(1, 16, 32), (3, 40, 96), (2, 64, 4096)])
def test_pack_int4_bit_exact(e4b, E, N, K):
    rng = np.random.default_rng(E * N + K)
    w = (0.02 * rng.standard_normal((E, N, K))).astype(np.float32)
    w[0, 0, :32] = 0.0                                     # an all-zero block
    w[-1, -1, 32 * (K // 32 - 1):] *= 1e-8                 # a block whose scale is tiny
    wb = f32_to_bf16_bits(w)
    packed, scales = e4b.e4b_pack_int4_b32(dev_bf16(wb))
    torch.cuda.synchronize()
    op, os_ = oi4.quantize_pack(wb)
    np.testing.assert_array_equal(host(packed), op)
    np.testing.assert_array_equal(_bits16(scales), os_)


@pytest.mark.parametrize("T,K", [(1, 32), (5, 2048), (3, 8192)])
def test_quantize_act_bit_exact(e4b, T, K):
    rng = np.random.default_rng(T + K)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[0, ::7] *= 100.0
    if T > 2:
        x[2] = 0.0                                         # an all-zero row
    xb = f32_to_bf16_bits(x)
    q, s = e4b.e4b_quantize_act_int8(dev_bf16(xb))
    torch.cuda.synchronize()
    oq, osx = oi4.quantize_act(xb)
    np.testing.assert_array_equal(host(q), oq)
    np.testing.assert_array_equal(host(s), osx)


def _routed_problem(E, N, K, T, k, seed):
    rng = np.random.default_rng(seed)
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((E, N, K))).astype(np.float32))
    x = f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return w, x, logits


@pytest.mark.parametrize("E,N,K,T,k", [
    (1, 16, 128, 1, 1),        # dense M = 1, one chunk per row
    (2, 32, 256, 2, 1),        # two tokens: the dot4 kernel's largest tile
    (2, 128, 256, 2, 1),       # dot4 kernel, K not split (one wave per 16 rows takes all of K)
    (3, 256, 1024, 3, 2),      # dot4 kernel, K split over 2 waves
    (5, 64, 512, 4, 2),        # four tokens: the MFMA kernel's smallest tile
    (3, 48, 256, 5, 2),        # ragged experts
    (4, 160, 640, 40, 2),      # experts with more than 16 routed rows: several token tiles
    (8, 256, 1024, 64, 8),     # every expert busy
    (2, 128, 8192, 3, 1),      # the largest K
    (4, 64, 8192, 20, 2),      # 16-row tiles at the largest K: 136 KB of LDS per workgroup
])
def test_int4_gemv_matches_oracle(e4b, E, N, K, T, k):
    w, x, logits = _routed_problem(E, N, K, T, k, seed=E * 100 + T)
    packed, scales = e4b.e4b_pack_int4_b32(dev_bf16(w))
    ids, tw, off, slots = e4b.e4b_route_permute(torch.from_numpy(logits).to(DEV), k)
    out = e4b.e4b_gemv_int4_b32(packed, scales, dev_bf16(x), k, off, slots)
    torch.cuda.synchronize()
    op, os_ = oi4.quantize_pack(w)
    ref, mag = oi4.grouped_gemv(op, os_, x, k, host(off), host(slots))
    got = host(out)
    assert np.all(np.isfinite(got))
    _assert_gemv_close(got, ref, mag, K, f"E={E} N={N} K={K} T={T} k={k}")


@pytest.mark.parametrize("E", [4096, 4100])
def test_int4_gemv_many_experts_hand_routed(e4b, E):
    """1-3 tokens run as one launch (tile lookup and activation quantisation inside the GEMV)
    up to 4096 experts, and as quantiser + GEMV launches above: both against the oracle, on a
    routing written by hand (the router takes at most 1024 experts), with an all-zero token."""
    N, K, T, k = 16, 128, 3, 2
    rng = np.random.default_rng(E)
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((E, N, K))).astype(np.float32))
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[1] = 0.0
    xb = f32_to_bf16_bits(x)
    ids = np.array([[5, E - 1], [5, 17], [E - 96, E - 1]])   # token t, choice j -> expert
    order = sorted(range(T * k), key=lambda s_: (ids.flat[s_], s_ // k))
    slots = np.array(order, np.int32)
    counts = np.bincount(ids.ravel(), minlength=E)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    packed, scales = e4b.e4b_pack_int4_b32(dev_bf16(w))
    out = e4b.e4b_gemv_int4_b32(packed, scales, dev_bf16(xb), k, torch.from_numpy(off).to(DEV),
                                torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    used = sorted(set(ids.ravel().tolist()))
    op, os_ = oi4.quantize_pack(w[used])
    off_u = np.concatenate([[0], np.cumsum(counts[used])]).astype(np.int32)
    ref, mag = oi4.grouped_gemv(op, os_, xb, k, off_u, slots)
    got = host(out)
    assert np.all(np.isfinite(got))
    _assert_gemv_close(got, ref, mag, K, f"E={E}")


def test_int4_gemv_is_deterministic(e4b):
    w, x, logits = _routed_problem(4, 128, 1024, 24, 2, 9)
    packed, scales = e4b.e4b_pack_int4_b32(dev_bf16(w))
    _, _, off, slots = e4b.e4b_route_permute(torch.from_numpy(logits).to(DEV), 2)
    a = e4b.e4b_gemv_int4_b32(packed, scales, dev_bf16(x), 2, off, slots)
    b = e4b.e4b_gemv_int4_b32(packed, scales, dev_bf16(x), 2, off, slots)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", list(INT4_WORKLOADS))
def test_int4_gemv_full_size_sampled_rows(e4b, name):
    """The stacks bench.py times (seeded bf16 weights packed on the GPU, the workload's routing
    of seeded logits); the oracle packs only the experts of the sampled rows, whose bytes and
    scales must also match the GPU's."""
    wl = INT4_WORKLOADS[name]
    N, K = 2 * wl.I, wl.H
    w = torch.empty((wl.E, N, K), dtype=torch.bfloat16, device=DEV)
    for e in range(wl.E):
        w[e].copy_(torch.from_numpy(make_expert_weight(wl, "gate_up", e).view(np.int16)).view(torch.bfloat16))
    packed, scales = e4b.e4b_pack_int4_b32(w)
    del w
    x = make_x(wl)
    _, _, off, slots = e4b.e4b_route_permute(torch.from_numpy(make_logits(wl)).to(DEV), wl.k)
    out = e4b.e4b_gemv_int4_b32(packed, scales, dev_bf16(x), wl.k, off, slots)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isfinite(got))
    offs, sl = host(off), host(slots)
    _, _, _, o_off, o_slots = oroute.route(make_logits(wl), wl.k)
    np.testing.assert_array_equal(offs, o_off)
    np.testing.assert_array_equal(sl, o_slots)
    rng = np.random.default_rng(17)
    S = wl.T * wl.k
    rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 6)]))
    experts = np.searchsorted(offs, rows, side="right") - 1
    op = np.zeros((wl.E, N, K // 2), np.uint8)
    os_ = np.zeros((wl.E, N, K // 32), np.uint16)
    for e in np.unique(experts):
        op[e], os_[e] = oi4.quantize_pack(make_expert_weight(wl, "gate_up", int(e)))
        np.testing.assert_array_equal(host(packed[e]), op[e])
        np.testing.assert_array_equal(_bits16(scales[e]), os_[e])
    ref, mag = oi4.grouped_gemv(op, os_, x, wl.k, offs, sl, rows=rows)
    _assert_gemv_close(got[rows], ref, mag[:], K, f"{name} rows {rows.tolist()}")
