"""GPU routing vs the oracle: ids, offsets and slots bit-exact, weights to float32 accuracy."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, host
from moe_inputs import DECODE_TOKENS, WORKLOADS, make_logits
from oracle import route as oroute

pytestmark = pytest.mark.gpu

W_RTOL = 2e-6  # float32 exp/sum/divide vs the float64 oracle


def _check(e4b, logits, k, renormalize=True):
    ids, w, off, slots = e4b.e4b_route_permute(torch.from_numpy(logits).to(DEV), k, renormalize)
    torch.cuda.synchronize()
    o_ids, o_w, _, o_off, o_slots = oroute.route(logits, k, renormalize)
    assert np.array_equal(host(ids), o_ids), "top-k ids differ"
    assert np.array_equal(host(off), o_off), "expert offsets differ"
    assert np.array_equal(host(slots), o_slots), "sorted slots differ"
    gw = host(w).astype(np.float64)
    assert np.all(np.abs(gw - o_w) <= W_RTOL * np.abs(o_w) + 1e-30), np.max(np.abs(gw - o_w) / o_w)
    return host(ids), host(off), host(slots)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_route_workloads(e4b, name):
    wl = WORKLOADS[name]
    Ts = DECODE_TOKENS if name == "finegrained_nf4_decode" else (wl.T,)
    for T in Ts:
        _check(e4b, make_logits(wl.with_T(T)), wl.k)


def test_route_skewed_has_empty_experts(e4b):
    wl = WORKLOADS["skewed_nf4_prefill"]
    _, off, _ = _check(e4b, make_logits(wl), wl.k)
    counts = np.diff(off)
    assert (counts == 0).sum() > 0 and counts.max() == wl.T


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 1, 1), (1, 8, 8), (33, 8, 8), (1, 128, 8),
                                   # up to 8 tokens: top-k folded into the one-launch router
                                   (8, 1024, 64), (8, 200, 5), (2, 65, 3), (6, 300, 64), (9, 128, 8),
                                   (300, 1024, 64), (70, 65, 3), (257, 16, 2),
                                   # several 1024-token chunks of the counting sort, ragged last
                                   (2500, 1024, 8), (3073, 3, 2), (1024, 7, 7), (1025, 1, 1),
                                   # chunk counts staged in LDS (9 x 910 = 8190 of at most 8192)
                                   # and read from memory (9 x 1024)
                                   (9000, 910, 2), (9000, 1024, 2)])
def test_route_edge_shapes(e4b, T, E, k):
    rng = np.random.default_rng(T * 1000 + E + k)
    _check(e4b, rng.standard_normal((T, E), dtype=np.float32), k)


def test_route_ties_and_signed_zero(e4b):
    rng = np.random.default_rng(2)
    lg = np.round(rng.standard_normal((200, 12)) * 2).astype(np.float32)  # many exact ties
    lg[0] = 0.0
    lg[1, ::2] = -0.0
    lg[2] = 1.0
    _check(e4b, lg, 4)
    _check(e4b, lg, 12)
    _check(e4b, lg[:6], 4)     # few tokens: the one-launch router


def test_route_without_renormalisation(e4b):
    rng = np.random.default_rng(3)
    _check(e4b, rng.standard_normal((64, 32), dtype=np.float32) * 3, 4, renormalize=False)
    _check(e4b, rng.standard_normal((3, 32), dtype=np.float32) * 3, 4, renormalize=False)


def test_route_empty_batch(e4b):
    ids, w, off, slots = e4b.e4b_route_permute(torch.zeros((0, 8), dtype=torch.float32, device=DEV), 2)
    torch.cuda.synchronize()
    assert np.array_equal(host(off), np.zeros(9, np.int32))


def test_route_is_deterministic(e4b):
    wl = WORKLOADS["skewed_nf4_prefill"]
    lg = torch.from_numpy(make_logits(wl)).to(DEV)
    a = [host(t) for t in e4b.e4b_route_permute(lg, wl.k)]
    b = [host(t) for t in e4b.e4b_route_permute(lg, wl.k)]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
