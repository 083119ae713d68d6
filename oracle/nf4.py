"""NF4 blockwise quantisation, packing and dequantisation (oracle; test infrastructure only).

Sources (project pages):
* bitsandbytes pull request #1984 "Experts4bit: fused MoE weights in 4-bit NF4/FP4",
  Summary and Design: every expert of a fused [E, N, K] stack is quantised on its own,
  stored as packed uint8 with float32 absmax, and dequantised on the fly.
* same page, Benchmark Results: NF4 error MAE 0.073 / RMSE 0.092 and ~28% of fp16 memory
  (these pin block 64; see the tests).
* grouped-nf4-gemm 0.25.0 project description, opening section: NF4 on the bitsandbytes
  gemm_4bit layout, decoded through a lookup table to fp32, then scaled per block.
* same page, "Try it on CPU right now", example 1: a [256, 512] weight packs to a
  [256, 256] uint8 array and a [256, 8] float32 absmax array (so the blocks run along K,
  64 wide, two codes per byte), re-packing the decoded weight reproduces the bytes.

Readings where the pages are silent (listed in the design notes):
* Codebook: the 16 NormalFloat-4 values published with QLoRA (Dettmers et al., 2023),
  held here as float32 bit patterns.
* Normalisation: n = float32(v / absmax), a correctly rounded float32 division.
* Code choice: the nearest codebook value to n; an exact tie goes to the lower code.
* All-zero block: absmax 0, every code 7 (the zero entry).
* Nibble order: within a byte, the even-indexed element sits in the high nibble.
* Decode: w = float32(C[code] * absmax), the float32 product of the table value and scale.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64

# NormalFloat-4 codebook (QLoRA, appendix E), float32 bit patterns, ascending.
NF4_CODEBOOK_BITS = np.array([
    0xBF800000, 0xBF3239B1, 0xBF066B30, 0xBECA32A0, 0xBE91A24D, 0xBE3D353F, 0xBDBA7871, 0x00000000,
    0x3DA2FAFF, 0x3E24CAE3, 0x3E7C04DD, 0x3EAD033A, 0x3EE1A4B8, 0x3F1007AB, 0x3F3913B3, 0x3F800000,
], dtype=np.uint32)
NF4_CODEBOOK = NF4_CODEBOOK_BITS.view(np.float32)


def _as_f32(w) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype == np.uint16:  # bf16 bit patterns
        return (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return w.astype(np.float32)


def nearest_code(n: np.ndarray) -> np.ndarray:
    """Index of the codebook value nearest to each float32 n; ties go to the lower code.

    Distances are taken in float64, where |n - C[c]| is exact for the float32 values
    involved at every tie, so an exact midpoint compares equal and argmin's first-minimum
    rule picks the lower code.
    """
    n32 = np.asarray(n, dtype=np.float32)
    flat = n32.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    cb = NF4_CODEBOOK.astype(np.float64)
    step = 1 << 20                       # bounded memory; element-wise, so chunking is exact
    for i in range(0, flat.size, step):
        d = np.abs(flat[i:i + step].astype(np.float64)[:, None] - cb)
        out[i:i + step] = np.argmin(d, axis=-1)
    return out.reshape(n32.shape)


def quantize_pack(w, block: int = BLOCK):
    """Quantise a weight [..., N, K] (bf16 bits or float) to NF4.

    Returns (packed uint8 [..., N, K/2], absmax float32 [..., N, K/block]).
    """
    v = _as_f32(w)
    K = v.shape[-1]
    if K % block:
        raise ValueError(f"K={K} is not a multiple of the block size {block}")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    a = np.max(np.abs(vb), axis=-1)                          # exact float32 max
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    n = (vb / safe[..., None]).astype(np.float32)            # float32 division, RNE
    codes = nearest_code(n)
    codes = np.where((a > 0)[..., None], codes, np.uint8(7))  # all-zero block -> zero code
    codes = codes.reshape(v.shape)
    packed = ((codes[..., 0::2] << 4) | codes[..., 1::2]).astype(np.uint8)
    return packed, a.astype(np.float32)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> codes [..., K] (even element from the high nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    codes[..., 0::2] = p >> 4
    codes[..., 1::2] = p & 0x0F
    return codes


def dequantize(packed: np.ndarray, absmax: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Decode to float32 [..., N, K]: float32(C[code] * absmax of the element's block)."""
    codes = unpack_codes(packed)
    K = codes.shape[-1]
    vals = NF4_CODEBOOK[codes]
    scale = np.repeat(np.asarray(absmax, np.float32), block, axis=-1)
    assert scale.shape[-1] == K
    return (vals * scale).astype(np.float32)


def bytes_per_element(block: int = BLOCK) -> float:
    """Storage per weight: 4 bits of code plus a float32 absmax shared by `block` weights."""
    return 0.5 + 4.0 / block
