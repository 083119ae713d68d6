"""Host-only checks of the C ABI: the library loads, exports every entry point that
include/e4b.h declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "e4b.h")
ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_OVERFLOW = -1, -2, -3, -4, -5, -6
FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(e4b_\w+)\s*\(", src, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("e4b_pack_nf4", "e4b_pack_mxfp4", "e4b_route_permute", "e4b_moe_forward",
              "e4b_route_workspace_bytes", "e4b_moe_workspace_bytes", "e4b_status_string", "e4b_version",
              "e4b_dgrad_workspace_bytes", "e4b_grouped_dgrad", "e4b_pack_int4_b32",
              "e4b_quantize_act_int8", "e4b_int4_gemv_workspace_bytes", "e4b_gemv_int4_b32",
              "e4b_moe_forward_noalloc", "e4b_noalloc_scratch_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(e4b):
    lib = ctypes.CDLL(e4b.lib_path)
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", e4b.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (e4b_\w+)", out))
    assert set(_declared()) <= exported


def test_version_and_status_strings(e4b):
    assert e4b.e4b_version() >= 100
    for s in range(-7, 1):
        assert e4b.e4b_status_string(s) and e4b.e4b_status_string(s) != "unknown status"


def _pack(e4b, fn, w=FAKE, E=2, N=4, K=128, o1=FAKE, o2=FAKE):
    c = e4b._c_pack_nf4 if fn == "nf4" else e4b._c_pack_mxfp4
    return c(w, E, N, K, o1, o2, None)


@pytest.mark.parametrize("fn,block", [("nf4", 64), ("mxfp4", 32)])
def test_pack_rejects_bad_arguments(e4b, fn, block):
    assert _pack(e4b, fn, w=None) == ERR_ARG
    assert _pack(e4b, fn, o1=None) == ERR_ARG
    assert _pack(e4b, fn, o2=None) == ERR_ARG
    assert _pack(e4b, fn, E=0) == ERR_ARG
    assert _pack(e4b, fn, N=-1) == ERR_ARG
    assert _pack(e4b, fn, K=block + block // 2) == ERR_SHAPE
    assert _pack(e4b, fn, w=FAKE + 8) == ERR_ALIGN
    assert _pack(e4b, fn, o1=FAKE + 4) == ERR_ALIGN
    assert _pack(e4b, fn, E=1 << 30, N=1 << 12, K=1 << 12) == ERR_OVERFLOW


def test_route_rejects_bad_arguments(e4b):
    def call(T=16, E=8, k=2, flags=1, ws_bytes=4096, **p):
        ptr = dict(logits=FAKE, ids=FAKE, w=FAKE, off=FAKE, slots=FAKE, ws=FAKE)
        ptr.update(p)
        return e4b._c_route(ptr["logits"], T, E, k, flags, ptr["ids"], ptr["w"], ptr["off"],
                            ptr["slots"], ptr["ws"], ws_bytes, None)
    assert call(k=0) == ERR_ARG
    assert call(k=9) == ERR_ARG
    assert call(E=0) == ERR_ARG
    assert call(T=-1) == ERR_ARG
    assert call(flags=2) == ERR_ARG
    assert call(E=2048, k=2) == ERR_SHAPE
    assert call(E=128, k=65) == ERR_SHAPE
    assert call(logits=None) == ERR_ARG
    assert call(off=None) == ERR_ARG
    assert call(ws=None) == ERR_ARG
    assert call(slots=FAKE + 2) == ERR_ALIGN
    assert call(ws_bytes=0) == ERR_WORKSPACE
    assert call(T=1 << 29, k=8) == ERR_OVERFLOW
    assert e4b.e4b_route_workspace_bytes(16, 8, 2) >= 32


def _args(e4b, **kw):
    a = e4b.MoeArgs()
    a.fmt, a.k, a.E, a.H, a.I, a.T = 0, 2, 8, 256, 512, 64
    for f in ("x", "w_gu", "s_gu", "w_dn", "s_dn", "topk_w", "expert_offsets", "sorted_slots", "out", "ws"):
        setattr(a, f, FAKE)
    a.out_f32 = None
    a.ws_bytes = 1 << 40
    a.flags = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_forward_rejects_bad_arguments(e4b):
    f = lambda **kw: e4b._c_moe_forward(ctypes.byref(_args(e4b, **kw)), None)
    assert f(fmt=2) == ERR_ARG
    assert f(k=0) == ERR_ARG
    assert f(k=9) == ERR_ARG
    assert f(E=0) == ERR_ARG
    assert f(T=-1) == ERR_ARG
    assert f(flags=3) == ERR_ARG
    assert f(flags=0x200) == ERR_ARG                 # unknown bit
    assert f(flags=0xC0) == ERR_ARG                  # both MXFP4 routes
    assert f(flags=0x40) not in (ERR_ARG, ERR_SHAPE)   # one MXFP4 route is accepted
    assert f(flags=0x30) not in (ERR_ARG, ERR_SHAPE)   # expert-variant bits are accepted
    assert f(flags=7) == ERR_ARG
    assert f(flags=0x6) == ERR_ARG                   # tile override with the streaming path
    assert f(H=96) == ERR_SHAPE
    assert f(I=100) == ERR_SHAPE
    assert f(x=None) == ERR_ARG
    assert f(s_dn=None) == ERR_ARG
    assert f(ws=None) == ERR_ARG
    assert f(out=FAKE + 2) == ERR_ALIGN
    assert f(out_f32=FAKE + 4) == ERR_ALIGN
    assert f(b_gu=FAKE + 4) == ERR_ALIGN
    assert f(b_dn=FAKE + 8) == ERR_ALIGN
    assert f(ws_bytes=1024) == ERR_WORKSPACE
    assert f(T=1 << 28, k=8) == ERR_OVERFLOW
    assert f(T=1 << 20, H=1 << 12) == ERR_OVERFLOW
    assert f(T=1, H=1 << 16, I=1 << 15) == ERR_OVERFLOW   # one expert's stack >= 2^31 bytes


def test_noalloc_forward_rejects_bad_arguments(e4b):
    """The allocation-free forward: same argument checks, no workspace argument, and a call that
    needs more than the fixed scratch is refused (all before any device is touched)."""
    f = lambda **kw: e4b._c_moe_forward_noalloc(ctypes.byref(_args(e4b, **kw)), None)
    assert e4b.e4b_noalloc_scratch_bytes() == 64 << 20
    assert f() == ERR_ARG                            # a workspace pointer is given
    assert f(ws=None, ws_bytes=0, fmt=2) == ERR_ARG
    assert f(ws=None, ws_bytes=0, H=96) == ERR_SHAPE
    assert f(ws=None, ws_bytes=0, out=FAKE + 2) == ERR_ALIGN
    assert f(ws=None, ws_bytes=0, T=1 << 16, k=8) == -8    # E4B_ERR_TOO_LARGE
    assert e4b.e4b_status_string(-8).startswith("the call needs more workspace")


def _dargs(e4b, **kw):
    a = e4b.DecodeArgs()
    a.fmt, a.k, a.E, a.H, a.I, a.T = 0, 8, 128, 2048, 768, 4
    for f in ("logits", "x", "w_gu", "s_gu", "w_dn", "s_dn", "out", "ws"):
        setattr(a, f, FAKE)
    a.ws_bytes = 1 << 40
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_step_rejects_bad_arguments(e4b):
    f = lambda **kw: e4b._c_decode_step(ctypes.byref(_dargs(e4b, **kw)), None)
    assert f(T=9) == ERR_SHAPE
    assert f(T=0) == ERR_SHAPE
    assert f(T=8, k=9) == ERR_SHAPE            # 72 routed slots
    assert f(E=1025, k=8) == ERR_SHAPE
    assert f(k=0) == ERR_ARG
    assert f(fmt=2) == ERR_ARG
    assert f(route_flags=2) == ERR_ARG
    assert f(flags=1) == ERR_ARG               # a path flag is not a decode-step flag
    assert f(reserved=1) == ERR_ARG
    assert f(H=96) == ERR_SHAPE
    assert f(x=None) == ERR_ARG
    assert f(ws=None) == ERR_ARG
    assert f(topk_ids=FAKE) == ERR_ARG         # ids without weights
    assert f(out=FAKE + 2) == ERR_ALIGN
    assert f(ws_bytes=1024) == ERR_WORKSPACE
    n = ctypes.c_size_t(0)
    assert e4b._c_decode_ws(ctypes.byref(_dargs(e4b)), ctypes.byref(n)) == 0
    assert n.value >= 256 + 4 * 8 * 768 * 2


def test_workspace_sizes_cover_the_intermediates(e4b):
    from moe_inputs import WORKLOADS
    for wl in WORKLOADS.values():
        n = e4b.e4b_moe_workspace_bytes(wl.fmt, wl.E, wl.H, wl.I, wl.T, wl.k)
        S = wl.T * wl.k
        assert n >= 2 * wl.T * wl.H + 2 * S * wl.I + 4 * S * wl.H
        assert n < 2 * (2 * wl.T * wl.H + 2 * S * wl.I + 4 * S * wl.H) + (1 << 20)
        # the atomic combine keeps its [T, H] float32 accumulator in the same layout
        na = e4b.e4b_moe_workspace_bytes(wl.fmt, wl.E, wl.H, wl.I, wl.T, wl.k, e4b.E4B_COMBINE_ATOMIC)
        assert na == n and na >= 4 * wl.T * wl.H


def test_dgrad_rejects_bad_arguments(e4b):
    def f(**kw):
        a = e4b.DgradArgs()
        a.fmt, a.E, a.N, a.K, a.S = 0, 4, 128, 256, 100
        for n in ("g", "w", "s", "expert_offsets", "out_f32", "ws"):
            setattr(a, n, FAKE)
        a.ws_bytes = 1 << 40
        for k, v in kw.items():
            setattr(a, k, v)
        return e4b._c_dgrad(ctypes.byref(a), None)
    assert f(fmt=3) == ERR_ARG
    assert f(E=0) == ERR_ARG
    assert f(S=-1) == ERR_ARG
    assert f(reserved=1) == ERR_ARG
    assert f(N=96) == ERR_SHAPE
    assert f(K=100) == ERR_SHAPE
    assert f(g=None) == ERR_ARG
    assert f(out_f32=None) == ERR_ARG
    assert f(out=FAKE + 2) == ERR_ALIGN
    assert f(ws_bytes=16) == ERR_WORKSPACE
    assert f(S=1 << 24, N=1 << 10) == ERR_OVERFLOW
    assert e4b.e4b_dgrad_workspace_bytes("nf4", 4, 128, 256, 100) >= 64


def test_int4_entry_points_reject_bad_arguments(e4b):
    pk = lambda w=FAKE, E=2, N=4, K=64, o1=FAKE, o2=FAKE: e4b._c_pack_int4(w, E, N, K, o1, o2, None)
    assert pk(w=None) == ERR_ARG
    assert pk(E=0) == ERR_ARG
    assert pk(K=48) == ERR_SHAPE
    assert pk(o2=FAKE + 2) == ERR_ALIGN
    qa = lambda x=FAKE, T=3, K=64, q=FAKE, s=FAKE: e4b._c_quant_act(x, T, K, q, s, None)
    assert qa(q=None) == ERR_ARG
    assert qa(T=-1) == ERR_ARG
    assert qa(K=40) == ERR_SHAPE
    assert qa(x=FAKE + 8) == ERR_ALIGN

    def f(**kw):
        a = e4b._int4_args(8, 256, 1024, 4, 2)
        for n in ("x", "w", "s", "expert_offsets", "sorted_slots", "out_f32", "ws"):
            setattr(a, n, FAKE)
        a.ws_bytes = 1 << 40
        for k, v in kw.items():
            setattr(a, k, v)
        return e4b._c_int4_gemv(ctypes.byref(a), None)
    assert f(E=0) == ERR_ARG
    assert f(k=0) == ERR_ARG
    assert f(k=9) == ERR_ARG
    assert f(T=-1) == ERR_ARG
    assert f(reserved=1) == ERR_ARG
    assert f(N=250) == ERR_SHAPE
    assert f(K=1000) == ERR_SHAPE
    assert f(K=8320) == ERR_SHAPE
    assert f(x=None) == ERR_ARG
    assert f(sorted_slots=FAKE + 4) == ERR_ALIGN
    assert f(ws_bytes=64) == ERR_WORKSPACE
    assert f(N=1 << 20, K=8192) == ERR_OVERFLOW
    n = e4b.e4b_int4_gemv_workspace_bytes(8, 256, 1024, 4, 2)
    assert n >= 4 * 1024 + 4 * 32 * 4 + 4 * 4
