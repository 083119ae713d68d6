"""Top-k routing and the expert-major slot order (oracle; test infrastructure only).

Sources (project pages):
* grouped-nf4-gemm 0.25.0 project description, opening paragraphs: one launch covers all
  active experts, and the package ships a router epilogue among its decode glue kernels;
  Cerin Amroth "ML systems" index, ownership list: swiglu and combine glue kernels.
* bitsandbytes pull request #1984, Design: the reference forward loops over experts, so
  each expert sees the tokens routed to it.

Readings where the pages are silent:
* Logits are float32 [T, E].  Each token takes the k largest logits, in descending order;
  equal logits are ordered by the lower expert index.
* Weights are the softmax over the chosen k logits (the full softmax renormalised over
  the top k).  With renormalisation off, they are the full softmax probabilities.
* A slot is s = t*k + j.  Slots are ordered expert-major, and by token within an expert;
  expert_offsets[e] is the exclusive prefix sum of the per-expert counts.
"""
from __future__ import annotations

import numpy as np


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k]: per token, experts by descending logit, ties to the lower index."""
    lg = np.asarray(logits, np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # A stable sort on the negated logits keeps equal logits in ascending expert order.
    order = np.argsort(-lg, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def softmax_weights(logits: np.ndarray, ids: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Routing weights in float64 [T, k]."""
    lg = np.asarray(logits, np.float64)
    chosen = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
    if renormalize:
        m = chosen.max(axis=1, keepdims=True)
        ex = np.exp(chosen - m)
        return ex / ex.sum(axis=1, keepdims=True)
    m = lg.max(axis=1, keepdims=True)
    return np.exp(chosen - m) / np.exp(lg - m).sum(axis=1, keepdims=True)


def permute(ids: np.ndarray, E: int):
    """(counts [E], expert_offsets [E+1], sorted_slots [T*k]) for the expert-major order."""
    T, k = ids.shape
    counts = np.bincount(ids.reshape(-1).astype(np.int64), minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    parts = []
    for e in range(E):
        t, j = np.nonzero(ids == e)          # row-major: tokens ascending
        parts.append(t.astype(np.int64) * k + j)
    slots = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return counts.astype(np.int32), offsets.astype(np.int32), slots.astype(np.int32)


def route(logits: np.ndarray, k: int, renormalize: bool = True):
    """Everything the router step produces: ids, weights (float64), counts, offsets, slots."""
    ids = topk(logits, k)
    w = softmax_weights(logits, ids, renormalize)
    counts, offsets, slots = permute(ids, np.asarray(logits).shape[1])
    return ids, w, counts, offsets, slots
