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

Expert variant of the MXFP4 family (experts4bit-qlora 0.35.0 project description, Scope:
MXFP4 experts with per-expert biases and a clamped GLU; the pages give no formula, so the
plainest reading is the released model family's own definition): gate and up rows interleaved (row
2j gate j, row 2j+1 up j), a bias on each gate_up row and on each down row, and
h = min(G, L) * sigmoid(a * min(G, L)) * (clip(U, -L, L) + 1) with L = 7 and a = 1.702
(g * sigmoid(1.702 g) is the sigmoid approximation of the Gaussian-error gate g * Phi(g)).
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


GLU_LIMIT = 7.0
GLU_ALPHA = 1.702


def clamped_glu(g: np.ndarray, u: np.ndarray, alpha: float = GLU_ALPHA,
                limit: float = GLU_LIMIT) -> np.ndarray:
    """min(g, limit) * sigmoid(alpha * min(g, limit)) * (clip(u, -limit, limit) + 1)."""
    gc = np.minimum(g, limit)
    uc = np.clip(u, -limit, limit)
    with np.errstate(over="ignore"):
        return gc / (1.0 + np.exp(-alpha * gc)) * (uc + 1.0)


def expert_mlp(x: np.ndarray, w_gu: np.ndarray, w_dn: np.ndarray, act: str = "swiglu",
               interleaved: bool = False, b_gu=None, b_dn=None) -> np.ndarray:
    """Expert MLP in float64: x [M, H], w_gu [2I, H], w_dn [H, I] -> [M, H].

    act "swiglu": silu(G) * U; "clamped_glu": clamped_glu(G, U).  Gate / up rows are the two
    halves of w_gu, or interleaved (even rows gate, odd rows up).  b_gu [2I] (same row order
    as w_gu) and b_dn [H] are added to the products when given.
    """
    I = w_dn.shape[1]
    gu = x @ w_gu.T
    if b_gu is not None:
        gu = gu + np.asarray(b_gu, np.float64)
    g, u = (gu[:, 0::2], gu[:, 1::2]) if interleaved else (gu[:, :I], gu[:, I:])
    h = silu(g) * u if act == "swiglu" else clamped_glu(g, u)
    y = h @ w_dn.T
    if b_dn is not None:
        y = y + np.asarray(b_dn, np.float64)
    return y


def forward(fmt: str, x_bits: np.ndarray, gu_packed, gu_scales, dn_packed, dn_scales,
            ids: np.ndarray, weights: np.ndarray, tokens=None, act: str = "swiglu",
            interleaved: bool = False, b_gu=None, b_dn=None, experts=None) -> np.ndarray:
    """out [len(tokens), H] float64 for the selected tokens (all tokens by default).

    Experts are visited one at a time; each expert's slice of the packed stacks is
    decoded and applied to the tokens (among the selected ones) routed to it.  act,
    interleaved, b_gu [E, 2I] and b_dn [E, H] select the expert variant (expert_mlp).
    `experts` (optional) restricts the sum to the slots routed to those experts, so the
    output over a partition of the experts is the sum of the partial outputs.
    """
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_bits_to_f64(np.asarray(x_bits)[tokens])
    H = x.shape[1]
    out = np.zeros((len(tokens), H), np.float64)
    sub_ids = np.asarray(ids)[tokens]
    sub_w = np.asarray(weights, np.float64)[tokens]
    for e in np.unique(sub_ids):
        if experts is not None and int(e) not in experts:
            continue
        rows, js = np.nonzero(sub_ids == e)
        w_gu = decode_expert(fmt, gu_packed, gu_scales, int(e))
        w_dn = decode_expert(fmt, dn_packed, dn_scales, int(e))
        y = expert_mlp(x[rows], w_gu, w_dn, act, interleaved,
                       None if b_gu is None else np.asarray(b_gu)[int(e)],
                       None if b_dn is None else np.asarray(b_dn)[int(e)])
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


def dgrad(fmt: str, packed: np.ndarray, scales: np.ndarray, g_bits: np.ndarray,
          offsets: np.ndarray) -> np.ndarray:
    """Grouped input gradient on the packed stacks, float64: for every expert e and each row p
    of its block [offsets[e], offsets[e+1]) of the grouped rows, out[p] = g[p] @ W_e, where
    W_e [N, K] is the decoded weight and g [S, N] the bf16 gradient of the expert's output.

    The transposed product of the forward step y = x W_e^T (Cerin Amroth "ML systems" index,
    Ownership: the kernels package owns the grouped packed GEMM and its dgrad): the same
    packed bytes, contracted over their row index N instead of K.
    """
    g = bf16_bits_to_f64(np.asarray(g_bits))
    S = g.shape[0]
    K = (packed.shape[2] * 2) if fmt == "nf4" else packed.shape[2] * 32
    out = np.zeros((S, K), np.float64)
    offsets = np.asarray(offsets, np.int64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = g[lo:hi] @ decode_expert(fmt, packed, scales, e)
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 (round to nearest even), returned as float32."""
    bits = f64_to_bf16_bits(np.asarray(a, np.float32).astype(np.float64))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def forward_dequant_bf16(fmt: str, x_bits: np.ndarray, gu_packed, gu_scales, dn_packed, dn_scales,
                         ids: np.ndarray, weights: np.ndarray, tokens=None, act: str = "swiglu",
                         interleaved: bool = False, b_gu=None, b_dn=None, experts=None) -> np.ndarray:
    """The unfused comparator of the fidelity claim (grouped-nf4-gemm 0.25.0 project
    description, "What is measured", first row: the fused path is more accurate than
    dequantise-to-bf16).  Each expert's weights are decoded and rounded to bf16, then used in
    bf16 matrix products with float32 accumulation whose results a bf16 framework returns in
    bf16: G and U (bias added before the rounding), h = act(G, U) computed from them and
    rounded to bf16, and Y (bias likewise).  The top-k weighted sum is float64.
    Arguments as `forward`; returns float64 [len(tokens), H].
    """
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    x = bf16_bits_to_f64(np.asarray(x_bits)[tokens]).astype(np.float32)
    H = x.shape[1]
    out = np.zeros((len(tokens), H), np.float64)
    sub_ids = np.asarray(ids)[tokens]
    sub_w = np.asarray(weights, np.float64)[tokens]
    for e in np.unique(sub_ids):
        if experts is not None and int(e) not in experts:
            continue
        rows, js = np.nonzero(sub_ids == e)
        w_gu = round_bf16(decode_expert(fmt, gu_packed, gu_scales, int(e)).astype(np.float32))
        w_dn = round_bf16(decode_expert(fmt, dn_packed, dn_scales, int(e)).astype(np.float32))
        I = w_dn.shape[1]
        gu = x[rows] @ w_gu.T
        if b_gu is not None:
            gu = gu + np.asarray(b_gu, np.float32)[int(e)]
        gu = round_bf16(gu)
        g, u = (gu[:, 0::2], gu[:, 1::2]) if interleaved else (gu[:, :I], gu[:, I:])
        g64, u64 = g.astype(np.float64), u.astype(np.float64)
        h = silu(g64) * u64 if act == "swiglu" else clamped_glu(g64, u64)
        h = round_bf16(h.astype(np.float32))
        y = h @ w_dn.T
        if b_dn is not None:
            y = y + np.asarray(b_dn, np.float32)[int(e)]
        y = round_bf16(y)
        out[rows] += sub_w[rows, js][:, None] * y.astype(np.float64)
    return out
