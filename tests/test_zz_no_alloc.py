"""The allocation-free entry point e4b_moe_forward_noalloc against e4b_moe_forward, through the
C ABI: two calls in a row on the library's fixed scratch, the second on a smaller layer, each
bit-identical to e4b_moe_forward on the same inputs (the same kernels run) and within the
per-row tolerance of the float64 oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_out_is_rne_of_f32, assert_rows_within_tolerance, host, random_layer

pytestmark = pytest.mark.gpu

# (fmt, E, H, I, T, k, path): the first call fills more of the scratch than the second
CALLS = [
    ("nf4", 32, 1024, 512, 64, 8, 0),     # streaming (decode) path, 512 routed rows
    ("mxfp4", 8, 256, 256, 5, 2, 1),      # MFMA tile path, 10 routed rows
]


def test_noalloc_matches_forward_on_two_calls(e4b):
    assert e4b.e4b_noalloc_scratch_bytes() == 64 << 20
    for i, (fmt, E, H, I, T, k, path) in enumerate(CALLS):
        lay = random_layer(e4b, fmt, E, H, I, T, k, seed=70 + i)
        ids, w, off, slots = lay.route()
        need = e4b.e4b_moe_workspace_bytes(fmt, E, H, I, T, k, path)
        assert need <= e4b.e4b_noalloc_scratch_bytes()
        out_a, f_a = e4b.e4b_moe_forward(fmt, lay.x, lay.gp, lay.gs, lay.dp, lay.ds, w, off, slots, k,
                                         out_f32=True, path=path)
        out_b = torch.full_like(out_a, 7.0)
        f_b = torch.full_like(f_a, 7.0)
        e4b.e4b_moe_forward_noalloc(fmt, lay.x, lay.gp, lay.gs, lay.dp, lay.ds, w, off, slots, k,
                                    out_b, f_b, path=path)
        torch.cuda.synchronize()
        print(f"call {i}: {fmt} E={E} H={H} I={I} T={T} k={k}, workspace {need} bytes", flush=True)
        assert np.array_equal(host(out_a), host(out_b))
        assert np.array_equal(host(f_a).view(np.uint32), host(f_b).view(np.uint32))
        assert_out_is_rne_of_f32(host(out_b), host(f_b))
        assert_rows_within_tolerance(host(f_b), lay.oracle_out(), f"noalloc call {i}")


def test_noalloc_refuses_a_workspace_argument_and_a_too_large_call(e4b):
    lay = random_layer(e4b, "nf4", 4, 256, 256, 8, 2, seed=9)
    ids, w, off, slots = lay.route()
    out = torch.empty((lay.T, lay.H), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        e4b.e4b_moe_forward_noalloc("nf4", lay.x, lay.gp, lay.gs, lay.dp, lay.ds, w, off, slots, 2, None)
    # through the C ABI directly: a workspace pointer is an argument error, and a layer whose
    # workspace exceeds the scratch is refused before anything is enqueued
    import ctypes
    a = e4b._moe_args("nf4", lay.x, lay.gp, lay.gs, lay.dp, lay.ds, w, off, slots, 4, 256, 256, 2,
                      out, None, torch.empty(1 << 20, dtype=torch.uint8, device="cuda:0"), 0)
    assert e4b._c_moe_forward_noalloc(ctypes.byref(a), None) == -1
    a.ws, a.ws_bytes = None, 0
    a.T = 1 << 20                       # 2M routed rows: far beyond 64 MiB of workspace
    assert e4b._c_moe_forward_noalloc(ctypes.byref(a), None) == -8
    torch.cuda.synchronize()
