"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through the C ABI,
and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from moe_inputs import f32_to_bf16_bits
from oracle import moe as omoe
from oracle import mxfp4 as omx
from oracle import nf4 as onf4
from oracle import route as oroute

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def oracle_pack(fmt: str, w_bits: np.ndarray):
    return (onf4 if fmt == "nf4" else omx).quantize_pack(w_bits)


def gpu_pack(e4b, fmt: str, w_dev: torch.Tensor):
    return e4b.e4b_pack_nf4(w_dev) if fmt == "nf4" else e4b.e4b_pack_mxfp4(w_dev)


def assert_rows_within_tolerance(got_f32: np.ndarray, ref: np.ndarray, what: str = ""):
    """Per row t: max |got - ref| <= 8e-3 * ||ref_t||_2 / sqrt(H) + 1e-3."""
    tau = omoe.tolerance(ref)
    err = np.max(np.abs(got_f32.astype(np.float64) - ref), axis=1)
    ratio = err / tau
    worst = int(np.argmax(ratio)) if len(ratio) else 0
    assert np.all(np.isfinite(got_f32)), f"{what}: non-finite output"
    assert np.all(ratio <= 1.0), (
        f"{what}: row {worst} err {err[worst]:.3e} > tol {tau[worst]:.3e} (ratio {ratio[worst]:.2f})")
    return float(ratio.max()) if len(ratio) else 0.0


def assert_out_is_rne_of_f32(out_bf16: np.ndarray, out_f32: np.ndarray):
    assert np.array_equal(out_bf16, f32_to_bf16_bits(out_f32))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_violations(out_bf16: np.ndarray, ref: np.ndarray):
    """The literal check of the bf16 output against the float64 reference, reported beside its
    floor: (elements of out_bf16 outside the per-row bound, elements of the bf16 rounding of ref
    itself outside it).  A bf16 half-ulp exceeds the bound for large |y|, so even a perfectly
    computed output has violations (the floor); the gate proper is on the fp32 output."""
    tau = omoe.tolerance(ref)[:, None]
    got = bf16_bits_to_f64(out_bf16)
    floor = bf16_bits_to_f64(f32_to_bf16_bits(ref.astype(np.float32)))
    return int(np.sum(np.abs(got - ref) > tau)), int(np.sum(np.abs(floor - ref) > tau))


class Layer:
    """Seeded inputs of one layer, on host (bits) and device; packed both ways."""

    def __init__(self, e4b, fmt, x_bits, logits, gu_bits, dn_bits, k):
        self.e4b, self.fmt, self.k = e4b, fmt, k
        self.x_bits, self.logits, self.gu_bits, self.dn_bits = x_bits, logits, gu_bits, dn_bits
        self.T, self.H = x_bits.shape
        self.E = gu_bits.shape[0]
        self.I = dn_bits.shape[2]
        self.x = dev_bf16(x_bits)
        self.logits_dev = torch.from_numpy(logits).to(DEV)
        gu = dev_bf16(gu_bits)
        dn = dev_bf16(dn_bits)
        self.gp, self.gs = gpu_pack(e4b, fmt, gu)
        self.dp, self.ds = gpu_pack(e4b, fmt, dn)
        del gu, dn

    def route(self, renormalize=True):
        return self.e4b.e4b_route_permute(self.logits_dev, self.k, renormalize)

    def forward(self, path=0, route=None, act="swiglu", interleaved=False, b_gu=None, b_dn=None):
        ids, w, off, slots = route if route is not None else self.route()
        dev = lambda b: None if b is None else torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(DEV)
        out, out32 = self.e4b.e4b_moe_forward(self.fmt, self.x, self.gp, self.gs, self.dp, self.ds,
                                              w, off, slots, self.k, out_f32=True, path=path,
                                              act=act, interleaved=interleaved,
                                              b_gu=dev(b_gu), b_dn=dev(b_dn))
        torch.cuda.synchronize()
        return host(out), host(out32)

    def oracle_out(self, tokens=None, act="swiglu", interleaved=False, b_gu=None, b_dn=None):
        gp, gs = oracle_pack(self.fmt, self.gu_bits)
        dp, ds = oracle_pack(self.fmt, self.dn_bits)
        ids, w, *_ = oroute.route(self.logits, self.k)
        # the GPU adds float32 biases: the oracle gets the same float32 values
        f32 = lambda b: None if b is None else np.asarray(b, np.float32).astype(np.float64)
        return omoe.forward(self.fmt, self.x_bits, gp, gs, dp, ds, ids, w, tokens, act=act,
                            interleaved=interleaved, b_gu=f32(b_gu), b_dn=f32(b_dn))


def random_layer(e4b, fmt, E, H, I, T, k, seed, wscale=0.02, logit_bias=None):
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    gu = f32_to_bf16_bits((wscale * rng.standard_normal((E, 2 * I, H))).astype(np.float32))
    dn = f32_to_bf16_bits((wscale * rng.standard_normal((E, H, I))).astype(np.float32))
    lg = rng.standard_normal((T, E), dtype=np.float32)
    if logit_bias is not None:
        lg = (lg + np.asarray(logit_bias, np.float32)[None, :]).astype(np.float32)
    return Layer(e4b, fmt, x, lg, gu, dn, k)
