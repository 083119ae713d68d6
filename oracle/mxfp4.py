"""MXFP4 quantisation, packing and dequantisation (oracle; test infrastructure only).

Sources (project pages):
* grouped-nf4-gemm 0.25.0 project description, opening section: MXFP4 is the OCP format,
  e2m1 elements sharing an e8m0 scale, used on a checkpoint's released bytes as they are.
* same page, "Try it on CPU right now", example 2: a [128, 256] weight packs to blocks
  [128, 8, 16] uint8 and scales [128, 8] uint8 (32 elements per scale, two per byte),
  with a round-trip relative error of about 0.12 on a normal weight.

The element and scale rules follow the OCP Microscaling Formats specification v1.0 (the
pages name the format, not the conversion):
* e2m1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
  subnormal (0 or 0.5).  Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* Shared scale of a 32-block: 2^(floor(log2(amax)) - 2), 2 being the largest e2m1
  exponent; clamped to the e8m0 range [-127, 127]; an all-zero block gets 2^-127
  (scale byte 0).  Byte = exponent + 127; the NaN byte 0xFF is never produced.
* Element: v / scale rounded to the nearest e2m1 magnitude, ties to the even code,
  magnitudes above 6 saturating to 6; the sign bit copies v's sign.
* Nibble order (released-checkpoint order): the even-indexed element is the low nibble.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def e2m1_value(code: int) -> float:
    """Value of a 4-bit e2m1 code from its bit fields (OCP MX v1.0, FP4 E2M1)."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = 0.5 * man                                  # subnormal: 2^(1-bias) * 0.m
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return sign * mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_MAG = E2M1[:8]


def _as_f32(w) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype == np.uint16:
        return (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return w.astype(np.float32)


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax == 0."""
    a = np.asarray(amax, np.float64)
    _, e = np.frexp(a)                 # a = m * 2^e, m in [0.5, 1)  =>  floor(log2 a) = e - 1
    s = (e.astype(np.int64) - 1) - 2
    s = np.clip(s, -127, 127)
    return np.where(a > 0, s, -127).astype(np.int64)


def round_e2m1_magnitude(q: np.ndarray) -> np.ndarray:
    """Nearest e2m1 magnitude code (0..7) of |q|; ties to the even code; saturate at 6."""
    m_all = np.abs(np.asarray(q, np.float64))
    flat = m_all.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    step = 1 << 20                       # bounded memory; element-wise, so chunking is exact
    for i in range(0, flat.size, step):
        m = flat[i:i + step]
        d = np.abs(m[:, None] - E2M1_MAG)                # exact for these dyadic values
        best = d.min(axis=-1, keepdims=True)
        cand = d == best
        # among equally near codes (at most two), take the even one
        even = cand & ((np.arange(8) % 2) == 0)
        pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
        out[i:i + step] = np.where(m >= 6.0, 7, pick)
    return out.reshape(m_all.shape)


def quantize_pack(w, block: int = BLOCK):
    """Quantise [..., N, K] to MXFP4: (blocks uint8 [..., N, K/32, 16], scales uint8 [..., N, K/32])."""
    v = _as_f32(w)
    K = v.shape[-1]
    if K % block:
        raise ValueError(f"K={K} is not a multiple of the block size {block}")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(vb), axis=-1)
    s = shared_exponent(amax)
    q = vb.astype(np.float64) / np.ldexp(1.0, s)[..., None]   # exact power-of-two scaling
    mag = round_e2m1_magnitude(q)
    sign = np.signbit(vb).astype(np.uint8) << 3
    codes = (mag | sign).astype(np.uint8)
    blocks = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (s + 127).astype(np.uint8)
    return blocks, scales


def unpack_codes(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, np.uint8)
    codes = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    codes[..., 0::2] = b & 0x0F
    codes[..., 1::2] = b >> 4
    return codes


def dequantize(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode to float32 [..., N, K]: e2m1 value times 2^(scale byte - 127) (exact)."""
    codes = unpack_codes(blocks)                       # [..., N, K/32, 32]
    vals = E2M1[codes] * np.ldexp(1.0, np.asarray(scales, np.int64) - 127)[..., None]
    out = vals.astype(np.float32)
    return out.reshape(out.shape[:-2] + (out.shape[-2] * out.shape[-1],))


def bytes_per_element(block: int = BLOCK) -> float:
    return 0.5 + 1.0 / block
