"""GPU packers vs the oracle: bytes and scales must match bit for bit."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev_bf16, gpu_pack, host, oracle_pack
from moe_inputs import WORKLOADS, f32_to_bf16_bits, make_expert_weight

pytestmark = pytest.mark.gpu


def _check(e4b, fmt, bits):
    p, s = gpu_pack(e4b, fmt, dev_bf16(bits))
    torch.cuda.synchronize()
    op, os_ = oracle_pack(fmt, bits)
    gp, gs = host(p), host(s)
    assert gp.shape == op.shape and gs.shape == os_.shape
    bad = np.argwhere(gp != op)
    assert bad.size == 0, f"{fmt}: {len(bad)} packed bytes differ, first at {bad[0]}"
    if fmt == "nf4":
        assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "absmax differs"
    else:
        assert np.array_equal(gs, os_), "scales differ"


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("shape", [(1, 1, 64), (3, 5, 128), (2, 7, 320), (4, 33, 1024)])
def test_pack_random_shapes(e4b, fmt, shape):
    rng = np.random.default_rng(sum(shape))
    bits = f32_to_bf16_bits((0.02 * rng.standard_normal(shape)).astype(np.float32))
    _check(e4b, fmt, bits)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_pack_every_bf16_value(e4b, fmt):
    """Every finite bf16 bit pattern, each in blocks with several different maxima, so every
    code boundary and every exponent is crossed (exhaustive edge coverage)."""
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allbits[((allbits.astype(np.uint32) >> 7) & 0xFF) != 0xFF]
    block = 64
    n = (len(finite) + block - 1) // block * block
    v = np.zeros(n, np.uint16)
    v[:len(finite)] = finite
    rows = [v]
    for amax in (1.0, 0.75, 3.0e-3, 1.0e30, 1.0e-30, 6.0):
        r = v.copy().reshape(-1, block)
        r[:, 0] = f32_to_bf16_bits(np.array([amax], np.float32))[0]
        rows.append(r.reshape(-1))
    bits = np.stack(rows)[None]                      # [1, rows, n]
    _check(e4b, fmt, bits)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_pack_zero_and_signed_zero_blocks(e4b, fmt):
    bits = np.zeros((2, 3, 128), np.uint16)
    bits[0, 1, :] = 0x8000                           # -0.0 everywhere
    bits[1, 2, 5] = 0x0001                           # one tiny subnormal
    _check(e4b, fmt, bits)


def test_pack_is_deterministic(e4b):
    rng = np.random.default_rng(9)
    w = dev_bf16(f32_to_bf16_bits(rng.standard_normal((4, 64, 512)).astype(np.float32)))
    a = [host(t) for t in e4b.e4b_pack_nf4(w)]
    b = [host(t) for t in e4b.e4b_pack_nf4(w)]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_pack_full_size_sampled_rows(e4b, name):
    """Whole expert stacks at the workload's real size are packed on the GPU; sampled rows
    (first, last and random) of sampled experts are checked against the oracle."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(1)
    experts = sorted({0, wl.E - 1, int(rng.integers(wl.E))})
    for which in ("gate_up", "down"):
        bits = np.stack([make_expert_weight(wl, which, e) for e in experts])
        p, s = gpu_pack(e4b, wl.fmt, dev_bf16(bits))
        torch.cuda.synchronize()
        gp, gs = host(p), host(s)
        N = bits.shape[1]
        rows = sorted({0, N - 1, *rng.integers(N, size=6).tolist()})
        op, os_ = oracle_pack(wl.fmt, bits[:, rows])
        assert np.array_equal(gp[:, rows], op)
        if wl.fmt == "nf4":
            assert np.array_equal(gs[:, rows].view(np.uint32), os_.view(np.uint32))
        else:
            assert np.array_equal(gs[:, rows], os_)
