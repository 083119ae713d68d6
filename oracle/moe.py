"""MoE layer forward in float64 on decoded 4-bit weights (oracle; test infrastructure only).

Sources (project pages):
* bitsandbytes pull request #1984, Summary and Design: fused expert stacks gate_up_proj
  and down_proj, dequantised per expert inside a loop over experts, SiLU-gated (SwiGLU)
  activation between the two projections.
* experts4bit-qlora 0.35.0 project description, opening section: transformers v5 keeps
  the experts as fused 3-D parameters gate_up_proj [E, 2I, H] and down_proj [E, H, I]
  (out x in).
* grouped-nf4-gemm 0.25.0 project description, opening section: table decode to fp32,
  block scaling, fp32 accumulation, bf16 epilogue; the oracle keeps every step after the
  decode in float64 with no intermediate rounding, as the exact result those steps
  approximate.
* Cerin Amroth "ML systems" index, ownership list: the combine step (top-k weighted sum).

Readings where the pages are silent:
* The first I rows of gate_up are the gate, the next I rows the up projection.
* h = silu(G) * U with silu(g) = g / (1 + exp(-g)); Y = h W_down^T; out[t] = sum over the
  token's k slots of weight * Y.
"""
from __future__ import annotations

import numpy as np

from . import mxfp4, nf4


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_expert(fmt: str, packed: np.ndarray, scales: np.ndarray, e: int) -> np.ndarray:
    """One expert's weight [N, K] as float64, decoded from its own packed slice."""
    if fmt == "nf4":
        return nf4.dequantize(packed[e], scales[e]).astype(np.float64)
    if fmt == "mxfp4":
        return mxfp4.dequantize(packed[e], scales[e]).astype(np.float64)
    raise ValueError(fmt)


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_mlp(x: np.ndarray, w_gu: np.ndarray, w_dn: np.ndarray) -> np.ndarray:
    """SwiGLU expert MLP in float64: x [M, H], w_gu [2I, H], w_dn [H, I] -> [M, H]."""
    I = w_dn.shape[1]
    g = x @ w_gu[:I].T
    u = x @ w_gu[I:].T
    return (silu(g) * u) @ w_dn.T


def forward(fmt: str, x_bits: np.ndarray, gu_packed, gu_scales, dn_packed, dn_scales,
            ids: np.ndarray, weights: np.ndarray, tokens=None) -> np.ndarray:
    """out [len(tokens), H] float64 for the selected tokens (all tokens by default).

    Experts are visited one at a time; each expert's slice of the packed stacks is
    decoded and applied to the tokens (among the selected ones) routed to it.
    """
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_bits_to_f64(np.asarray(x_bits)[tokens])
    H = x.shape[1]
    out = np.zeros((len(tokens), H), np.float64)
    sub_ids = np.asarray(ids)[tokens]
    sub_w = np.asarray(weights, np.float64)[tokens]
    for e in np.unique(sub_ids):
        rows, js = np.nonzero(sub_ids == e)
        w_gu = decode_expert(fmt, gu_packed, gu_scales, int(e))
        w_dn = decode_expert(fmt, dn_packed, dn_scales, int(e))
        y = expert_mlp(x[rows], w_gu, w_dn)
        out[rows] += sub_w[rows, js][:, None] * y
    return out


def tolerance(ref_rows: np.ndarray) -> np.ndarray:
    """Per-row bound on |gpu - oracle|: 8e-3 * ||row||_2 / sqrt(H) + 1e-3."""
    ref = np.asarray(ref_rows, np.float64)
    H = ref.shape[-1]
    return 8e-3 * np.linalg.norm(ref, axis=-1) / np.sqrt(H) + 1e-3


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 -> bfloat16 bits (via float32, each step round-to-nearest-even)."""
    u = np.asarray(a, np.float64).astype(np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)
