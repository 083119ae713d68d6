"""int4-b32 weights, int8 activations and the integer decode GEMV (oracle; test infrastructure
only).

Sources (project pages):
* grouped-nf4-gemm 0.25.0 project description, opening section: besides the grouped GEMM the
  package carries an int4-b32 decode GEMV and a calibrated packer for it.
* Cerin Amroth "ML systems" index, Solutions: a single-token int4-b32 decode GEMV over routed
  MoE experts with exact integer accumulation; calibrated (GPTQ) weights are packed onto the
  same bytes.
* grouped-nf4-gemm 0.25.0 project description, What is measured: the dense M = 1 int4-b32
  decode GEMV is quoted in GB/s of weight streaming.

The pages name the format and the exact integer accumulation and nothing else.  Readings
(listed in the design notes):
* int4-b32: signed 4-bit integer codes q in [-8, 7] (two's complement nibbles), one scale per
  32 consecutive weights of a row; round-to-nearest packing (the calibrated GPTQ packer needs
  calibration data and is not built): s = fp16(absmax / 7) (float32 division, correctly
  rounded, then round-to-nearest-even to fp16), q = clamp(rint(w / s), -8, 7) with the float32
  division by the stored scale; an all-zero block (or one whose scale rounds to 0) gets s = 0
  and q = 0.  Weight = s * q.
* Nibble order: the even-indexed element in the low nibble (the GPTQ int32 packing order read
  byte by byte).
* Integer accumulation needs integer activations: each token's activation row is quantised to
  int8 with one float32 scale per token, s_x = absmax / 127 (float32, correctly rounded),
  q_x = clamp(rint(x / s_x), -127, 127); an all-zero row gets s_x = 0 and q_x = 0.
* Output: y[n] = s_x * sum_b s[n, b] * I_b, where I_b = sum over the block's 32 k of
  q[n, k] * q_x[k] is an exact integer; the oracle takes the block sums in exact integers
  and the rest in float64.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
QMAX_W = 7
QMAX_X = 127


def _as_f32(w) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype == np.uint16:  # bf16 bit patterns
        return (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return w.astype(np.float32)


def quantize_pack(w, block: int = BLOCK):
    """Round-to-nearest int4-b32 packing of a weight [..., N, K] (bf16 bits or float).

    Returns (packed uint8 [..., N, K/2], scales fp16 bit patterns uint16 [..., N, K/32]).
    """
    v = _as_f32(w)
    K = v.shape[-1]
    if K % block:
        raise ValueError(f"K={K} is not a multiple of the block size {block}")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    a = np.max(np.abs(vb), axis=-1)                                  # exact float32 max
    s16 = (a / np.float32(QMAX_W)).astype(np.float32).astype(np.float16)  # f32 div, RNE to fp16
    s = s16.astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((vb / safe[..., None]).astype(np.float32))           # float32 division, RNE
    q = np.clip(q, -8, QMAX_W)
    q = np.where((s > 0)[..., None], q, 0).astype(np.int8).reshape(v.shape)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, s16.view(np.uint16)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> signed codes int8 [..., K] (even element from the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    nib = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int16)
    nib[..., 0::2] = p & 0x0F
    nib[..., 1::2] = p >> 4
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


def scales_f64(scales_bits: np.ndarray) -> np.ndarray:
    return np.asarray(scales_bits, np.uint16).view(np.float16).astype(np.float64)


def dequantize(packed: np.ndarray, scales_bits: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Decode to float64 [..., N, K]: s * q (exact in float64)."""
    q = unpack_codes(packed).astype(np.float64)
    s = np.repeat(scales_f64(scales_bits), block, axis=-1)
    assert s.shape == q.shape
    return q * s


def quantize_act(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-token int8 quantisation of activations [T, K] (bf16 bits or float).

    Returns (q_x int8 [T, K], s_x float32 [T])."""
    v = _as_f32(x)
    a = np.max(np.abs(v), axis=-1)
    s = (a / np.float32(QMAX_X)).astype(np.float32)                  # float32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((v / safe[:, None]).astype(np.float32))
    q = np.clip(q, -QMAX_X, QMAX_X)
    q = np.where((s > 0)[:, None], q, 0).astype(np.int8)
    return q, s


def block_sums(codes: np.ndarray, qx: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Exact integer block dot products I[n, b] = sum_{k in block b} q[n, k] * q_x[k] for one
    token: codes int8 [N, K], qx int8 [K] -> int64 [N, K/block]."""
    prod = codes.astype(np.int64) * qx.astype(np.int64)[None, :]
    N, K = prod.shape
    return prod.reshape(N, K // block, block).sum(axis=-1)


def gemv_rows(packed: np.ndarray, scales_bits: np.ndarray, qx: np.ndarray,
              sx: float) -> tuple[np.ndarray, np.ndarray]:
    """One token through one expert: y[n] = s_x * sum_b s[n, b] * I_b (float64), and the
    float64 sum of the terms' magnitudes s_x * sum_b |s[n, b] * I_b| (the scale of the
    rounding error of any float32 evaluation of the same sum)."""
    I = block_sums(unpack_codes(packed), qx)
    terms = scales_f64(scales_bits) * I.astype(np.float64)
    return float(sx) * terms.sum(axis=-1), float(sx) * np.abs(terms).sum(axis=-1)


def grouped_gemv(packed: np.ndarray, scales_bits: np.ndarray, x, k: int, offsets, slots,
                 rows=None) -> tuple[np.ndarray, np.ndarray]:
    """The routed decode GEMV: for every sorted row p of expert e (offsets from the router),
    token t = slots[p] // k, y[p] = W_e x_t in the integer form above.  `rows` limits the
    evaluation to some sorted rows (default: all).  Returns (y float64 [len(rows), N], the
    magnitude sums of gemv_rows)."""
    qx, sx = quantize_act(x)
    offsets = np.asarray(offsets, np.int64)
    slots = np.asarray(slots, np.int64)
    rows = np.arange(len(slots)) if rows is None else np.asarray(rows, np.int64)
    N = packed.shape[-2]
    y = np.zeros((len(rows), N))
    mag = np.zeros((len(rows), N))
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    for i, p in enumerate(rows):
        e, t = int(expert_of[i]), int(slots[p] // k)
        y[i], mag[i] = gemv_rows(packed[e], scales_bits[e], qx[t], sx[t])
    return y, mag


def bytes_per_element(block: int = BLOCK) -> float:
    return 0.5 + 2.0 / block
