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
    "E4B_ROUTE_RENORMALIZE", "E4B_ACT_CLAMPED_GLU", "E4B_GU_INTERLEAVED", "lib_path", "e4b_version", "e4b_status_string", "e4b_pack_nf4",
    "e4b_pack_mxfp4", "e4b_route_workspace_bytes", "e4b_route_permute", "e4b_moe_workspace_bytes",
    "e4b_moe_forward", "MoeArgs", "e4b_dgrad_workspace_bytes", "e4b_grouped_dgrad", "DgradArgs",
]

E4B_FMT_NF4, E4B_FMT_MXFP4 = 0, 1
E4B_PATH_AUTO, E4B_PATH_GEMM, E4B_PATH_GEMV = 0, 1, 2
E4B_TILE_AUTO, E4B_TILE_32, E4B_TILE_128, E4B_TILE_256 = 0x0, 0x4, 0x8, 0xC
E4B_ROUTE_RENORMALIZE = 1
E4B_ACT_CLAMPED_GLU, E4B_GU_INTERLEAVED = 0x10, 0x20
_FMT = {"nf4": E4B_FMT_NF4, "mxfp4": E4B_FMT_MXFP4, E4B_FMT_NF4: E4B_FMT_NF4, E4B_FMT_MXFP4: E4B_FMT_MXFP4}

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libe4b.so")
if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is not built; build it with `python -m bit_quantized_mixture_amd.build` "
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


def _need(t, name, dtypes, shape=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
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
    E, N, K = w.shape
    if packed is None:
        packed = torch.empty((E, N, K // 2), dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty((E, N, K // 64), dtype=torch.float32, device=w.device)
    _need(packed, "packed", (torch.uint8,), (E, N, K // 2))
    _need(absmax, "absmax", (torch.float32,), (E, N, K // 64))
    _check("e4b_pack_nf4", _c_pack_nf4(_ptr(w), E, N, K, _ptr(packed), _ptr(absmax), _stream(stream)))
    return packed, absmax


def e4b_pack_mxfp4(w, blocks=None, scales=None, stream=None):
    """w [E, N, K] bf16 -> (blocks uint8 [E, N, K/32, 16], scales uint8 [E, N, K/32])."""
    _need(w, "w", _BF16)
    E, N, K = w.shape
    if blocks is None:
        blocks = torch.empty((E, N, K // 32, 16), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=w.device)
    _need(blocks, "blocks", (torch.uint8,), (E, N, K // 32, 16))
    _need(scales, "scales", (torch.uint8,), (E, N, K // 32))
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
    T, E = logits.shape
    dev = logits.device
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        slots = torch.empty((T * k,), dtype=torch.int32, device=dev)
    else:
        ids, w, offsets, slots = out
        _need(ids, "topk_ids", (torch.int32,), (T, k))
        _need(w, "topk_w", (torch.float32,), (T, k))
        _need(offsets, "expert_offsets", (torch.int32,), (E + 1,))
        _need(slots, "sorted_slots", (torch.int32,), (T * k,))
    if ws is None:
        need = e4b_route_workspace_bytes(T, E, k)
        ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
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
    """
    _need(x, "x", _BF16)
    T, H = x.shape
    E = expert_offsets.numel() - 1
    I = w_dn.shape[2] * (2 if w_dn.dim() == 3 else 32)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if out_f32 is True:
        out_f32 = torch.empty((T, H), dtype=torch.float32, device=dev)
    if ws is None:
        need = e4b_moe_workspace_bytes(fmt, E, H, I, T, k, path)
        ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    if act not in ("swiglu", "clamped_glu"):
        raise ValueError(f"act must be 'swiglu' or 'clamped_glu', not {act!r}")
    flags = path | (E4B_ACT_CLAMPED_GLU if act == "clamped_glu" else 0) | (E4B_GU_INTERLEAVED if interleaved else 0)
    for name, b, n in (("b_gu", b_gu, (E, 2 * I)), ("b_dn", b_dn, (E, H))):
        if b is not None:
            _need(b, name, (torch.float32,), n)
    a = _moe_args(fmt, x, w_gu, s_gu, w_dn, s_dn, topk_w, expert_offsets, sorted_slots, E, H, I, k,
                  out, out_f32, ws, flags)
    a.b_gu = None if b_gu is None else b_gu.data_ptr()
    a.b_dn = None if b_dn is None else b_dn.data_ptr()
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events needs 6 events")
        handles = (_vp * 6)(*[ev.cuda_event for ev in stage_events])
        a.stage_events = ctypes.cast(handles, ctypes.POINTER(_vp))
    _check("e4b_moe_forward", _c_moe_forward(ctypes.byref(a), _stream(stream)))
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
    S, N = g.shape
    E = w.shape[0]
    K = w.shape[2] * (2 if w.dim() == 3 else 32)
    if w.shape[1] != N:
        raise ValueError(f"w has {w.shape[1]} rows per expert, g has {N} columns")
    _need(expert_offsets, "expert_offsets", (torch.int32,), (E + 1,))
    dev = g.device
    if out_f32 is None:
        out_f32 = torch.empty((S, K), dtype=torch.float32, device=dev)
    if out is True:
        out = torch.empty((S, K), dtype=torch.bfloat16, device=dev)
    elif out is False:
        out = None
    if ws is None:
        ws = torch.empty((max(e4b_dgrad_workspace_bytes(fmt, E, N, K, S), 256),), dtype=torch.uint8, device=dev)
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
    E, N, K = w.shape
    if packed is None:
        packed = torch.empty((E, N, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((E, N, K // 32), dtype=torch.float16, device=w.device)
    _check("e4b_pack_int4_b32", _c_pack_int4(_ptr(w), E, N, K, _ptr(packed), _ptr(scales), _stream(stream)))
    return packed, scales


def e4b_quantize_act_int8(x, stream=None):
    """x [T, K] bf16 -> (q int8 [T, K], s float32 [T]): per-token int8 activations."""
    _need(x, "x", _BF16)
    T, K = x.shape
    q = torch.empty((T, K), dtype=torch.int8, device=x.device)
    sc = torch.empty((max(T, 1),), dtype=torch.float32, device=x.device)[:T]
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
    if out is None:
        out = torch.empty((T * k, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty((max(e4b_int4_gemv_workspace_bytes(E, N, K, T, k), 256),),
                         dtype=torch.uint8, device=x.device)
    a = _int4_args(E, N, K, T, k)
    a.x, a.w, a.s = x.data_ptr(), w.data_ptr(), s.data_ptr()
    a.expert_offsets, a.sorted_slots = expert_offsets.data_ptr(), sorted_slots.data_ptr()
    a.out_f32 = out.data_ptr()
    a.ws, a.ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    _check("e4b_gemv_int4_b32", _c_int4_gemv(ctypes.byref(a), _stream(stream)))
    return out
