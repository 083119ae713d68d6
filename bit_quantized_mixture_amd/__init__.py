"""Python binding of the e4b C ABI (include/e4b.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are torch CUDA
(HIP) tensors used purely as device memory; every step of the computation runs in the HIP
kernels of libe4b.so.  There is no fallback: if the library is missing, importing this
package raises, and if a call fails, E4BError is raised with the library's status.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "E4BError", "E4B_FMT_NF4", "E4B_FMT_MXFP4", "E4B_PATH_AUTO", "E4B_PATH_GEMM", "E4B_PATH_GEMV",
    "E4B_ROUTE_RENORMALIZE", "E4B_ACT_CLAMPED_GLU", "E4B_GU_INTERLEAVED", "E4B_MXFP4_SCALED", "E4B_MXFP4_FP16", "E4B_COMBINE_ATOMIC", "lib_path", "e4b_version", "e4b_status_string", "e4b_pack_nf4",
    "e4b_pack_mxfp4", "e4b_route_workspace_bytes", "e4b_route_permute", "e4b_moe_workspace_bytes",
    "e4b_moe_forward", "e4b_moe_forward_noalloc", "e4b_noalloc_scratch_bytes", "e4b_stream_probe", "e4b_decode_workspace_bytes", "e4b_moe_decode_step", "MoeArgs", "e4b_dgrad_workspace_bytes", "e4b_grouped_dgrad", "DgradArgs",
]

E4B_FMT_NF4, E4B_FMT_MXFP4 = 0, 1
E4B_PATH_AUTO, E4B_PATH_GEMM, E4B_PATH_GEMV = 0, 1, 2
E4B_TILE_AUTO, E4B_TILE_32, E4B_TILE_128, E4B_TILE_256 = 0x0, 0x4, 0x8, 0xC
E4B_ROUTE_RENORMALIZE = 1
E4B_ACT_CLAMPED_GLU, E4B_GU_INTERLEAVED = 0x10, 0x20
E4B_MXFP4_SCALED, E4B_MXFP4_FP16 = 0x40, 0x80
E4B_COMBINE_ATOMIC = 0x100
_FMT = {"nf4": E4B_FMT_NF4, "mxfp4": E4B_FMT_MXFP4, E4B_FMT_NF4: E4B_FMT_NF4, E4B_FMT_MXFP4: E4B_FMT_MXFP4}

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libe4b.so")
if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is not built; build it with `python bit_quantized_mixture_amd/build.py` "
        "(hipcc, gfx950).  There is no non-HIP implementation.")
_lib = ctypes.CDLL(lib_path)

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class MoeArgs(ctypes.Structure):
    """Mirror of struct e4b_moe_args."""
    _fields_ = [
        ("fmt", _i32), ("k", _i32), ("E", _i64), ("H", _i64), ("I", _i64), ("T", _i64),
        ("x", _vp), ("w_gu", _vp), ("s_gu", _vp), ("w_dn", _vp), ("s_dn", _vp),
        ("topk_w", _vp), ("expert_offsets", _vp), ("sorted_slots", _vp),
        ("out", _vp), ("out_f32", _vp), ("ws", _vp), ("ws_bytes", _sz),
        ("flags", _i32), ("reserved", _i32), ("stage_events", ctypes.POINTER(_vp)),
        ("b_gu", _vp), ("b_dn", _vp),
    ]


class DecodeArgs(ctypes.Structure):
    """Mirror of struct e4b_decode_args."""
    _fields_ = [
        ("fmt", _i32), ("k", _i32), ("E", _i64), ("H", _i64), ("I", _i64), ("T", _i64),
        ("route_flags", _i32), ("flags", _i32),
        ("logits", _vp), ("x", _vp), ("w_gu", _vp), ("s_gu", _vp), ("w_dn", _vp), ("s_dn", _vp),
        ("b_gu", _vp), ("b_dn", _vp), ("topk_ids", _vp), ("topk_w", _vp), ("expert_offsets", _vp),
        ("sorted_slots", _vp), ("out", _vp), ("out_f32", _vp), ("status", _vp),
        ("spin_limit", _i32), ("reserved", _i32), ("ws", _vp), ("ws_bytes", _sz),
    ]


class DgradArgs(ctypes.Structure):
    """Mirror of struct e4b_dgrad_args."""
    _fields_ = [
        ("fmt", _i32), ("reserved", _i32), ("E", _i64), ("N", _i64), ("K", _i64), ("S", _i64),
        ("g", _vp), ("w", _vp), ("s", _vp), ("expert_offsets", _vp), ("out_f32", _vp), ("out", _vp),
        ("ws", _vp), ("ws_bytes", _sz),
    ]


class Int4GemvArgs(ctypes.Structure):
    """Mirror of struct e4b_int4_gemv_args."""
    _fields_ = [
        ("E", _i64), ("N", _i64), ("K", _i64), ("T", _i64), ("k", _i32), ("reserved", _i32),
        ("x", _vp), ("w", _vp), ("s", _vp), ("expert_offsets", _vp), ("sorted_slots", _vp),
        ("out_f32", _vp), ("ws", _vp), ("ws_bytes", _sz),
    ]


def _decl(name, argtypes, restype=ctypes.c_int):
    fn = getattr(_lib, name)
    fn.argtypes = argtypes
    fn.restype = restype
    return fn


_c_version = _decl("e4b_version", [])
_c_status_string = _decl("e4b_status_string", [ctypes.c_int], ctypes.c_char_p)
_c_pack_nf4 = _decl("e4b_pack_nf4", [_vp, _i64, _i64, _i64, _vp, _vp, _vp])
_c_pack_mxfp4 = _decl("e4b_pack_mxfp4", [_vp, _i64, _i64, _i64, _vp, _vp, _vp])
_c_route_ws = _decl("e4b_route_workspace_bytes", [_i64, _i64, _i32, ctypes.POINTER(_sz)])
_c_route = _decl("e4b_route_permute", [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_c_moe_ws = _decl("e4b_moe_workspace_bytes", [ctypes.POINTER(MoeArgs), ctypes.POINTER(_sz)])
_c_moe_forward = _decl("e4b_moe_forward", [ctypes.POINTER(MoeArgs), _vp])
_c_moe_forward_noalloc = _decl("e4b_moe_forward_noalloc", [ctypes.POINTER(MoeArgs), _vp])
_c_noalloc_bytes = _decl("e4b_noalloc_scratch_bytes", [], _sz)
_c_stream_probe = _decl("e4b_stream_probe", [_vp, _vp, _i64, _i32, _vp])
_c_decode_ws = _decl("e4b_decode_workspace_bytes", [ctypes.POINTER(DecodeArgs), ctypes.POINTER(_sz)])
_c_decode_step = _decl("e4b_moe_decode_step", [ctypes.POINTER(DecodeArgs), _vp])
_c_dgrad_ws = _decl("e4b_dgrad_workspace_bytes", [ctypes.POINTER(DgradArgs), ctypes.POINTER(_sz)])
_c_dgrad = _decl("e4b_grouped_dgrad", [ctypes.POINTER(DgradArgs), _vp])
_c_pack_int4 = _decl("e4b_pack_int4_b32", [_vp, _i64, _i64, _i64, _vp, _vp, _vp])
_c_quant_act = _decl("e4b_quantize_act_int8", [_vp, _i64, _i64, _vp, _vp, _vp])
_c_int4_ws = _decl("e4b_int4_gemv_workspace_bytes", [ctypes.POINTER(Int4GemvArgs), ctypes.POINTER(_sz)])
_c_int4_gemv = _decl("e4b_gemv_int4_b32", [ctypes.POINTER(Int4GemvArgs), _vp])


class E4BError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({e4b_status_string(status)})")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise E4BError(fn, status)


def e4b_version() -> int:
    return _c_version()


def e4b_status_string(status: int) -> str:
    return _c_status_string(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class _on_stream:
    """Context for the binding's own allocations (outputs and workspaces it creates): they are
    made on the stream the kernels run on, so the caching allocator does not hand the memory to
    other work before those kernels are done.  A raw stream handle (not a torch stream) other
    than the current stream cannot be tracked: the caller then passes every buffer."""

    def __init__(self, stream):
        self.stream = stream
        self.ctx = None

    def __enter__(self):
        s = self.stream
        if s is None:
            return self
        if isinstance(s, torch.cuda.Stream):
            self.ctx = torch.cuda.stream(s)
            self.ctx.__enter__()
        elif int(s) != torch.cuda.current_stream().cuda_stream:
            self.ctx = False
        return self

    def alloc(self, *a, **kw):
        if self.ctx is False:
            raise ValueError("pass a torch.cuda.Stream, or preallocate every output and workspace, "
                             "when the work runs on a raw stream handle other than the current stream")
        return torch.empty(*a, **kw)

    def __exit__(self, *exc):
        if self.ctx:
            self.ctx.__exit__(*exc)
        return False


def _need(t, name, dtypes, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor, not {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_BF16 = (torch.bfloat16, torch.uint16, torch.int16)


def e4b_pack_nf4(w, packed=None, absmax=None, stream=None):
    """w [E, N, K] bf16 -> (packed uint8 [E, N, K/2], absmax float32 [E, N, K/64])."""
    _need(w, "w", _BF16)
    if w.dim() != 3:
        raise ValueError(f"w must be [E, N, K], got shape {tuple(w.shape)}")
    E, N, K = w.shape
    with _on_stream(stream) as st:
        if packed is None:
            packed = st.alloc((E, N, K // 2), dtype=torch.uint8, device=w.device)
        if absmax is None:
            absmax = st.alloc((E, N, K // 64), dtype=torch.float32, device=w.device)
    _need(packed, "packed", (torch.uint8,), (E, N, K // 2), w.device)
    _need(absmax, "absmax", (torch.float32,), (E, N, K // 64), w.device)
    _check("e4b_pack_nf4", _c_pack_nf4(_ptr(w), E, N, K, _ptr(packed), _ptr(absmax), _stream(stream)))
    return packed, absmax


def e4b_pack_mxfp4(w, blocks=None, scales=None, stream=None):
    """w [E, N, K] bf16 -> (blocks uint8 [E, N, K/32, 16], scales uint8 [E, N, K/32])."""
    _need(w, "w", _BF16)
    if w.dim() != 3:
        raise ValueError(f"w must be [E, N, K], got shape {tuple(w.shape)}")
    E, N, K = w.shape
    with _on_stream(stream) as st:
        if blocks is None:
            blocks = st.alloc((E, N, K // 32, 16), dtype=torch.uint8, device=w.device)
        if scales is None:
            scales = st.alloc((E, N, K // 32), dtype=torch.uint8, device=w.device)
    _need(blocks, "blocks", (torch.uint8,), (E, N, K // 32, 16), w.device)
    _need(scales, "scales", (torch.uint8,), (E, N, K // 32), w.device)
    _check("e4b_pack_mxfp4", _c_pack_mxfp4(_ptr(w), E, N, K, _ptr(blocks), _ptr(scales), _stream(stream)))
    return blocks, scales


def e4b_route_workspace_bytes(T: int, E: int, k: int) -> int:
    n = _sz(0)
    _check("e4b_route_workspace_bytes", _c_route_ws(T, E, k, ctypes.byref(n)))
    return n.value


def e4b_route_permute(logits, k: int, renormalize: bool = True, ws=None, stream=None, out=None):
    """logits [T, E] float32 -> (topk_ids [T,k] i32, topk_w [T,k] f32, expert_offsets [E+1] i32,
    sorted_slots [T*k] i32).  `out`: optional preallocated (ids, w, offsets, slots)."""
    _need(logits, "logits", (torch.float32,))
    if logits.dim() != 2:
        raise ValueError(f"logits must be [T, E], got shape {tuple(logits.shape)}")
    T, E = logits.shape
    dev = logits.device
    with _on_stream(stream) as st:
        if out is None:
            out = (st.alloc((T, k), dtype=torch.int32, device=dev),
                   st.alloc((T, k), dtype=torch.float32, device=dev),
                   st.alloc((E + 1,), dtype=torch.int32, device=dev),
                   st.alloc((T * k,), dtype=torch.int32, device=dev))
        if ws is None:
            need = e4b_route_workspace_bytes(T, E, k)
            ws = st.alloc((max(need, 256),), dtype=torch.uint8, device=dev)
    ids, w, offsets, slots = out
    _need(ids, "topk_ids", (torch.int32,), (T, k), dev)
    _need(w, "topk_w", (torch.float32,), (T, k), dev)
    _need(offsets, "expert_offsets", (torch.int32,), (E + 1,), dev)
    _need(slots, "sorted_slots", (torch.int32,), (T * k,), dev)
    _need(ws, "ws", (torch.uint8,), device=dev)
    flags = E4B_ROUTE_RENORMALIZE if renormalize else 0
    _check("e4b_route_permute", _c_route(
        _ptr(logits), T, E, k, flags, _ptr(ids), _ptr(w), _ptr(offsets), _ptr(slots),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return ids, w, offsets, slots


def _moe_args(fmt, x, w_gu, s_gu, w_dn, s_dn, topk_w, expert_offsets, sorted_slots, E, H, I, k,
              out, out_f32, ws, path) -> MoeArgs:
    a = MoeArgs()
    a.fmt = _FMT[fmt]
    a.k, a.E, a.H, a.I = k, E, H, I
    a.T = 0 if x is None else x.shape[0]
    for name, t in (("x", x), ("w_gu", w_gu), ("s_gu", s_gu), ("w_dn", w_dn), ("s_dn", s_dn),
                    ("topk_w", topk_w), ("expert_offsets", expert_offsets),
                    ("sorted_slots", sorted_slots), ("out", out), ("out_f32", out_f32), ("ws", ws)):
        setattr(a, name, None if t is None else t.data_ptr())
    a.ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    a.flags = path
    return a


def e4b_moe_workspace_bytes(fmt, E: int, H: int, I: int, T: int, k: int, path: int = E4B_PATH_AUTO) -> int:
    a = MoeArgs()
    a.fmt, a.k, a.E, a.H, a.I, a.T, a.flags = _FMT[fmt], k, E, H, I, T, path
    n = _sz(0)
    _check("e4b_moe_workspace_bytes", _c_moe_ws(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def _stack_shapes(fmt: int, E: int, N: int, K: int):
    """(codes shape, codes dtype, scales shape, scales dtype) of a packed [E, N, K] stack."""
    if fmt == E4B_FMT_NF4:
        return (E, N, K // 2), torch.uint8, (E, N, K // 64), torch.float32
    return (E, N, K // 32, 16), torch.uint8, (E, N, K // 32), torch.uint8


def e4b_moe_forward(fmt, x, w_gu, s_gu, w_dn, s_dn, topk_w, expert_offsets, sorted_slots, k: int,
                    out=None, out_f32=None, ws=None, path: int = E4B_PATH_AUTO, stream=None,
                    stage_events=None, act: str = "swiglu", interleaved: bool = False,
                    b_gu=None, b_dn=None):
    """MoE expert layer on packed weights.  Returns (out bf16 [T, H], out_f32 or None).

    `out_f32`: pass True to allocate the float32 output, a tensor to fill it, None to skip.
    `act` "swiglu" or "clamped_glu", `interleaved` gate/up row order, `b_gu` [E, 2I] and
    `b_dn` [E, H] float32 biases (or None): the expert variant flags of include/e4b.h.
    `stage_events`: None, or 6 torch.cuda.Event (enable_timing=True), each recorded once
    beforehand so that it exists; the call records them around its 5 stages.
    Every tensor is checked (device, dtype, contiguity, the shape implied by fmt, E, H, I, T, k)
    before the library is called.
    """
    return _moe_forward_call(_c_moe_forward, "e4b_moe_forward", fmt, x, w_gu, s_gu, w_dn, s_dn,
                             topk_w, expert_offsets, sorted_slots, k, out, out_f32, ws, path, stream,
                             stage_events, act, interleaved, b_gu, b_dn)


def _moe_forward_call(cfn, cname, fmt, x, w_gu, s_gu, w_dn, s_dn, topk_w, expert_offsets,
                      sorted_slots, k, out, out_f32, ws, path, stream, stage_events, act,
                      interleaved, b_gu, b_dn):
    noalloc = cfn is _c_moe_forward_noalloc
    if fmt not in _FMT:
        raise ValueError(f"fmt must be 'nf4' or 'mxfp4', not {fmt!r}")
    f = _FMT[fmt]
    _need(x, "x", _BF16)
    dev = x.device
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got shape {tuple(x.shape)}")
    T, H = x.shape
    _need(expert_offsets, "expert_offsets", (torch.int32,), device=dev)
    if expert_offsets.dim() != 1 or expert_offsets.numel() < 2:
        raise ValueError("expert_offsets must be [E + 1] with E >= 1")
    E = expert_offsets.numel() - 1
    _need(w_dn, "w_dn", (torch.uint8,), device=dev)
    if f == E4B_FMT_NF4 and w_dn.dim() == 3:
        I = w_dn.shape[2] * 2
    elif f == E4B_FMT_MXFP4 and w_dn.dim() == 4 and w_dn.shape[3] == 16:
        I = w_dn.shape[2] * 32
    else:
        raise ValueError(f"w_dn of shape {tuple(w_dn.shape)} is not a {fmt} down stack")
    for name, t, (N, K) in (("gate_up", (w_gu, s_gu), (2 * I, H)), ("down", (w_dn, s_dn), (H, I))):
        cs, cd, ss, sd = _stack_shapes(f, E, N, K)
        _need(t[0], f"w_{name}", (cd,), cs, dev)
        _need(t[1], f"s_{name}", (sd,), ss, dev)
    _need(topk_w, "topk_w", (torch.float32,), (T, k), dev)
    _need(sorted_slots, "sorted_slots", (torch.int32,), (T * k,), dev)
    if act not in ("swiglu", "clamped_glu"):
        raise ValueError(f"act must be 'swiglu' or 'clamped_glu', not {act!r}")
    for name, b, n in (("b_gu", b_gu, (E, 2 * I)), ("b_dn", b_dn, (E, H))):
        if b is not None:
            _need(b, name, (torch.float32,), n, dev)
    with _on_stream(stream) as st:
        if out is None:
            out = st.alloc((T, H), dtype=torch.bfloat16, device=dev)
        if out_f32 is True:
            out_f32 = st.alloc((T, H), dtype=torch.float32, device=dev)
        if ws is None and not noalloc:
            need = e4b_moe_workspace_bytes(fmt, E, H, I, T, k, path)
            ws = st.alloc((max(need, 256),), dtype=torch.uint8, device=dev)
    _need(out, "out", _BF16, (T, H), dev)
    if out_f32 is not None:
        _need(out_f32, "out_f32", (torch.float32,), (T, H), dev)
    if not noalloc:
        _need(ws, "ws", (torch.uint8,), device=dev)
    flags = path | (E4B_ACT_CLAMPED_GLU if act == "clamped_glu" else 0) | (E4B_GU_INTERLEAVED if interleaved else 0)
    a = _moe_args(fmt, x, w_gu, s_gu, w_dn, s_dn, topk_w, expert_offsets, sorted_slots, E, H, I, k,
                  out, out_f32, ws, flags)
    a.b_gu = None if b_gu is None else b_gu.data_ptr()
    a.b_dn = None if b_dn is None else b_dn.data_ptr()
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events needs 6 events")
        handles = (_vp * 6)(*[ev.cuda_event for ev in stage_events])
        a.stage_events = ctypes.cast(handles, ctypes.POINTER(_vp))
    _check(cname, cfn(ctypes.byref(a), _stream(stream)))
    return out, out_f32


def _dgrad_args(fmt, E, N, K, S) -> DgradArgs:
    a = DgradArgs()
    a.fmt, a.E, a.N, a.K, a.S = _FMT[fmt], E, N, K, S
    return a


def e4b_dgrad_workspace_bytes(fmt, E: int, N: int, K: int, S: int) -> int:
    n = _sz(0)
    _check("e4b_dgrad_workspace_bytes", _c_dgrad_ws(ctypes.byref(_dgrad_args(fmt, E, N, K, S)), ctypes.byref(n)))
    return n.value


def e4b_grouped_dgrad(fmt, g, w, s, expert_offsets, out_f32=None, out=False, ws=None, stream=None):
    """Grouped dgrad on a packed stack: out[p] = g[p] @ W_e for the rows p of expert e.

    g: [S, N] bf16 (rows grouped by expert); w, s: a packed stack as returned by
    e4b_pack_nf4 / e4b_pack_mxfp4 ([E, N, K/2] | [E, N, K/32, 16] and its scales);
    expert_offsets [E+1] int32.  Returns (out_f32 [S, K], out bf16 [S, K] or None); pass
    out=True to get the bf16 copy.
    """
    _need(g, "g", _BF16)
    if g.dim() != 2:
        raise ValueError(f"g must be [S, N], got shape {tuple(g.shape)}")
    S, N = g.shape
    if w.dim() not in (3, 4):
        raise ValueError(f"w of shape {tuple(w.shape)} is not a packed stack")
    E = w.shape[0]
    K = w.shape[2] * (2 if w.dim() == 3 else 32)
    if w.shape[1] != N:
        raise ValueError(f"w has {w.shape[1]} rows per expert, g has {N} columns")
    dev = g.device
    _need(expert_offsets, "expert_offsets", (torch.int32,), (E + 1,), dev)
    cs, cd, ss, sd = _stack_shapes(_FMT[fmt], E, N, K)
    _need(w, "w", (cd,), cs, dev)
    _need(s, "s", (sd,), ss, dev)
    with _on_stream(stream) as st:
        if out_f32 is None:
            out_f32 = st.alloc((S, K), dtype=torch.float32, device=dev)
        if out is True:
            out = st.alloc((S, K), dtype=torch.bfloat16, device=dev)
        elif out is False:
            out = None
        if ws is None:
            ws = st.alloc((max(e4b_dgrad_workspace_bytes(fmt, E, N, K, S), 256),), dtype=torch.uint8, device=dev)
    _need(out_f32, "out_f32", (torch.float32,), (S, K), dev)
    if out is not None:
        _need(out, "out", _BF16, (S, K), dev)
    _need(ws, "ws", (torch.uint8,), device=dev)
    a = _dgrad_args(fmt, E, N, K, S)
    a.g, a.w, a.s, a.expert_offsets = g.data_ptr(), w.data_ptr(), s.data_ptr(), expert_offsets.data_ptr()
    a.out_f32 = out_f32.data_ptr()
    a.out = None if out is None else out.data_ptr()
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    _check("e4b_grouped_dgrad", _c_dgrad(ctypes.byref(a), _stream(stream)))
    return out_f32, out


def e4b_pack_int4_b32(w, packed=None, scales=None, stream=None):
    """w [E, N, K] bf16 -> (packed uint8 [E, N, K/2], scales float16 [E, N, K/32])."""
    _need(w, "w", _BF16)
    if w.dim() != 3:
        raise ValueError(f"w must be [E, N, K], got shape {tuple(w.shape)}")
    E, N, K = w.shape
    with _on_stream(stream) as st:
        if packed is None:
            packed = st.alloc((E, N, K // 2), dtype=torch.uint8, device=w.device)
        if scales is None:
            scales = st.alloc((E, N, K // 32), dtype=torch.float16, device=w.device)
    _need(packed, "packed", (torch.uint8,), (E, N, K // 2), w.device)
    _need(scales, "scales", (torch.float16, torch.int16), (E, N, K // 32), w.device)
    _check("e4b_pack_int4_b32", _c_pack_int4(_ptr(w), E, N, K, _ptr(packed), _ptr(scales), _stream(stream)))
    return packed, scales


def e4b_quantize_act_int8(x, stream=None):
    """x [T, K] bf16 -> (q int8 [T, K], s float32 [T]): per-token int8 activations."""
    _need(x, "x", _BF16)
    if x.dim() != 2:
        raise ValueError(f"x must be [T, K], got shape {tuple(x.shape)}")
    T, K = x.shape
    with _on_stream(stream) as st:
        q = st.alloc((T, K), dtype=torch.int8, device=x.device)
        sc = st.alloc((max(T, 1),), dtype=torch.float32, device=x.device)[:T]
    _check("e4b_quantize_act_int8", _c_quant_act(_ptr(x), T, K, _ptr(q), _ptr(sc), _stream(stream)))
    return q, sc


def _int4_args(E, N, K, T, k):
    a = Int4GemvArgs()
    a.E, a.N, a.K, a.T, a.k, a.reserved = E, N, K, T, k, 0
    return a


def e4b_int4_gemv_workspace_bytes(E: int, N: int, K: int, T: int, k: int) -> int:
    n = _sz(0)
    _check("e4b_int4_gemv_workspace_bytes",
           _c_int4_ws(ctypes.byref(_int4_args(E, N, K, T, k)), ctypes.byref(n)))
    return n.value


def e4b_gemv_int4_b32(w, s, x, k: int, expert_offsets, sorted_slots, out=None, ws=None, stream=None):
    """Routed int4-b32 decode GEMV with exact integer accumulation.

    w [E, N, K/2] uint8 and s [E, N, K/32] float16 from e4b_pack_int4_b32; x [T, K] bf16;
    expert_offsets [E+1] and sorted_slots [T*k] int32 from e4b_route_permute.  Returns
    out [T*k, N] float32 in sorted-row order (row p: token sorted_slots[p] // k through the
    expert whose offsets contain p).
    """
    _need(x, "x", _BF16)
    T, K = x.shape
    _need(w, "w", (torch.uint8,))
    E, N = w.shape[0], w.shape[1]
    _need(w, "w", (torch.uint8,), (E, N, K // 2))
    _need(s, "s", (torch.float16, torch.int16), (E, N, K // 32))
    _need(expert_offsets, "expert_offsets", (torch.int32,), (E + 1,))
    _need(sorted_slots, "sorted_slots", (torch.int32,), (T * k,))
    with _on_stream(stream) as st:
        if out is None:
            out = st.alloc((T * k, N), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = st.alloc((max(e4b_int4_gemv_workspace_bytes(E, N, K, T, k), 256),),
                          dtype=torch.uint8, device=x.device)
    _need(out, "out", (torch.float32,), (T * k, N), x.device)
    _need(ws, "ws", (torch.uint8,), device=x.device)
    a = _int4_args(E, N, K, T, k)
    a.x, a.w, a.s = x.data_ptr(), w.data_ptr(), s.data_ptr()
    a.expert_offsets, a.sorted_slots = expert_offsets.data_ptr(), sorted_slots.data_ptr()
    a.out_f32 = out.data_ptr()
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    _check("e4b_gemv_int4_b32", _c_int4_gemv(ctypes.byref(a), _stream(stream)))
    return out


def e4b_noalloc_scratch_bytes() -> int:
    return _c_noalloc_bytes()


def e4b_moe_forward_noalloc(fmt, x, w_gu, s_gu, w_dn, s_dn, topk_w, expert_offsets, sorted_slots,
                            k: int, out, out_f32=None, path: int = E4B_PATH_AUTO, stream=None,
                            act: str = "swiglu", interleaved: bool = False, b_gu=None, b_dn=None):
    """e4b_moe_forward without a workspace argument and without any allocation: the library's
    fixed device scratch is the workspace.  `out` (bf16 [T, H]) must be given; `out_f32`
    (float32 [T, H]) may be.  Raises E4BError (E4B_ERR_TOO_LARGE) when the call needs more
    workspace than the scratch holds.  Calls that overlap on one GPU race on the scratch."""
    if out is None:
        raise ValueError("e4b_moe_forward_noalloc allocates nothing: pass `out`")
    if out_f32 is True:
        raise ValueError("e4b_moe_forward_noalloc allocates nothing: pass an out_f32 tensor or None")
    return _moe_forward_call(_c_moe_forward_noalloc, "e4b_moe_forward_noalloc", fmt, x, w_gu, s_gu,
                             w_dn, s_dn, topk_w, expert_offsets, sorted_slots, k, out, out_f32, None,
                             path, stream, None, act, interleaved, b_gu, b_dn)


def e4b_stream_probe(src, dst=None, stream=None):
    """Plain streaming read of `src` (dst None) or copy src -> dst: the measured memory ceiling
    beside the layer's rates.  Tensors must be contiguous device tensors of equal byte size."""
    _need(src, "src", (src.dtype,))
    nbytes = src.numel() * src.element_size()
    if dst is not None:
        _need(dst, "dst", (dst.dtype,), device=src.device)
        if dst.numel() * dst.element_size() != nbytes:
            raise ValueError("dst must have the byte size of src")
    _check("e4b_stream_probe", _c_stream_probe(_ptr(src), _ptr(dst), nbytes, 0 if dst is None else 1,
                                               _stream(stream)))


def _decode_args(fmt, E, H, I, T, k) -> DecodeArgs:
    a = DecodeArgs()
    a.fmt, a.k, a.E, a.H, a.I, a.T = _FMT[fmt], k, E, H, I, T
    return a


def e4b_decode_workspace_bytes(fmt, E: int, H: int, I: int, T: int, k: int) -> int:
    n = _sz(0)
    _check("e4b_decode_workspace_bytes",
           _c_decode_ws(ctypes.byref(_decode_args(fmt, E, H, I, T, k)), ctypes.byref(n)))
    return n.value


def e4b_moe_decode_step(fmt, logits, x, w_gu, s_gu, w_dn, s_dn, k: int, renormalize: bool = True,
                        out=None, out_f32=None, ws=None, route_out=None, status=None,
                        spin_limit: int = 0, act: str = "swiglu", interleaved: bool = False,
                        b_gu=None, b_dn=None, stream=None):
    """Routing + expert layer for T <= 8 tokens in one launch.  Returns (out, out_f32, route)
    where route is (topk_ids, topk_w, expert_offsets, sorted_slots) or None.

    `out_f32`: True to allocate, a tensor, or None.  `route_out`: True to allocate the routing
    outputs, a 4-tuple of tensors to fill, or None.  `ws`: a uint8 device tensor of at least
    e4b_decode_workspace_bytes(), zero-filled before its first use (allocated
    here with zeros when not given); keep it for later calls.  `status`: an int32 [1] device
    tensor that receives 0, or 1 if the kernel's grid barrier gave up waiting.
    """
    if fmt not in _FMT:
        raise ValueError(f"fmt must be 'nf4' or 'mxfp4', not {fmt!r}")
    f = _FMT[fmt]
    _need(x, "x", _BF16)
    dev = x.device
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got shape {tuple(x.shape)}")
    T, H = x.shape
    _need(logits, "logits", (torch.float32,), device=dev)
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError(f"logits must be [T, E] with T = {T}, got shape {tuple(logits.shape)}")
    E = logits.shape[1]
    _need(w_dn, "w_dn", (torch.uint8,), device=dev)
    if f == E4B_FMT_NF4 and w_dn.dim() == 3:
        I = w_dn.shape[2] * 2
    elif f == E4B_FMT_MXFP4 and w_dn.dim() == 4 and w_dn.shape[3] == 16:
        I = w_dn.shape[2] * 32
    else:
        raise ValueError(f"w_dn of shape {tuple(w_dn.shape)} is not a {fmt} down stack")
    for name, t, (N, K) in (("gate_up", (w_gu, s_gu), (2 * I, H)), ("down", (w_dn, s_dn), (H, I))):
        cs, cd, ss, sd = _stack_shapes(f, E, N, K)
        _need(t[0], f"w_{name}", (cd,), cs, dev)
        _need(t[1], f"s_{name}", (sd,), ss, dev)
    for name, b, n in (("b_gu", b_gu, (E, 2 * I)), ("b_dn", b_dn, (E, H))):
        if b is not None:
            _need(b, name, (torch.float32,), n, dev)
    if act not in ("swiglu", "clamped_glu"):
        raise ValueError(f"act must be 'swiglu' or 'clamped_glu', not {act!r}")
    with _on_stream(stream) as st:
        if out is None:
            out = st.alloc((T, H), dtype=torch.bfloat16, device=dev)
        if out_f32 is True:
            out_f32 = st.alloc((T, H), dtype=torch.float32, device=dev)
        if route_out is True:
            route_out = (st.alloc((T, k), dtype=torch.int32, device=dev),
                         st.alloc((T, k), dtype=torch.float32, device=dev),
                         st.alloc((E + 1,), dtype=torch.int32, device=dev),
                         st.alloc((T * k,), dtype=torch.int32, device=dev))
        if ws is None:
            if st.ctx is False:
                st.alloc(0)  # raises: a raw foreign stream needs a caller workspace
            ws = torch.zeros((max(e4b_decode_workspace_bytes(fmt, E, H, I, T, k), 256),),
                             dtype=torch.uint8, device=dev)
    _need(out, "out", _BF16, (T, H), dev)
    if out_f32 is not None:
        _need(out_f32, "out_f32", (torch.float32,), (T, H), dev)
    if route_out is not None:
        for name, t, dt, shp in zip(("topk_ids", "topk_w", "expert_offsets", "sorted_slots"), route_out,
                                    (torch.int32, torch.float32, torch.int32, torch.int32),
                                    ((T, k), (T, k), (E + 1,), (T * k,))):
            _need(t, name, (dt,), shp, dev)
    if status is not None:
        _need(status, "status", (torch.int32,), (1,), dev)
    _need(ws, "ws", (torch.uint8,), device=dev)
    a = _decode_args(fmt, E, H, I, T, k)
    a.route_flags = E4B_ROUTE_RENORMALIZE if renormalize else 0
    a.flags = (E4B_ACT_CLAMPED_GLU if act == "clamped_glu" else 0) | (E4B_GU_INTERLEAVED if interleaved else 0)
    a.logits, a.x = logits.data_ptr(), x.data_ptr()
    a.w_gu, a.s_gu, a.w_dn, a.s_dn = w_gu.data_ptr(), s_gu.data_ptr(), w_dn.data_ptr(), s_dn.data_ptr()
    a.b_gu = None if b_gu is None else b_gu.data_ptr()
    a.b_dn = None if b_dn is None else b_dn.data_ptr()
    if route_out is not None:
        a.topk_ids, a.topk_w, a.expert_offsets, a.sorted_slots = (t.data_ptr() for t in route_out)
    a.out = out.data_ptr()
    a.out_f32 = None if out_f32 is None else out_f32.data_ptr()
    a.status = None if status is None else status.data_ptr()
    a.spin_limit = spin_limit
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    _check("e4b_moe_decode_step", _c_decode_step(ctypes.byref(a), _stream(stream)))
    return out, out_f32, route_out
