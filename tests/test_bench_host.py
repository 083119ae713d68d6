"""Host logic of bench.py (no GPU): the roofline entry, the storage cost per weight, the
kernel-source hash that keys the committed HBM counters, and the one-GPU guard."""
import glob
import hashlib
import os
import re
import subprocess
import sys

import pytest

import bench
from moe_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bytes_per_weight_is_the_formats_storage():
    # NF4: a 4-bit code plus one fp32 absmax per 64 weights; MXFP4: a 4-bit code plus one
    # 8-bit e8m0 scale per 32
    assert bench.bytes_per_weight("nf4") == pytest.approx((4 + 32 / 64) / 8)
    assert bench.bytes_per_weight("mxfp4") == pytest.approx((4 + 8 / 32) / 8)


def _stages(gu_ms, dn_ms):
    return {"stage_ms": {"convert_x": 0.01, "build_tiles": 0.005, "gemm_gate_up": gu_ms,
                         "gemm_down": dn_ms, "combine": 0.02}}


def test_roofline_prefill_is_mfma_bound_on_the_slower_stage():
    wl = WORKLOADS["skewed_nf4_prefill"]
    S = wl.T * wl.k
    r = bench.roofline(wl, wl.E, _stages(3.0, 2.0), {"gemm_gate_up": 1.5e9})
    assert r["bound"] == "mfma" and r["kernel"] == "gemm_gate_up" and r["unit"] == "TFLOP/s"
    flops = 2 * S * (2 * wl.I) * wl.H                   # one multiply-add per weight and row
    assert r["algorithmic_flops"] == pytest.approx(flops)
    assert r["achieved"] == pytest.approx(flops / 3.0e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0)
    assert r["traffic"] == 1.5e9
    r = bench.roofline(wl, wl.E, _stages(1.0, 2.0), {})
    assert r["kernel"] == "gemm_down" and r["traffic"] is None
    assert r["algorithmic_flops"] == pytest.approx(2 * S * wl.I * wl.H)


def test_roofline_decode_is_hbm_bound_on_the_weight_bytes():
    wl = WORKLOADS["finegrained_nf4_decode"]
    assert wl.T * wl.k / wl.E < 16
    n_active = 100
    r = bench.roofline(wl, n_active, _stages(0.05, 0.03), None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["traffic"] is None
    wbytes = n_active * 2 * wl.I * wl.H * 0.5625
    abytes = 2 * wl.T * wl.H + 2 * wl.T * wl.k * wl.I
    assert r["algorithmic_bytes"] == pytest.approx(wbytes + abytes)
    assert r["achieved"] == pytest.approx((wbytes + abytes) / 0.05e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)


def test_kernel_source_hash_covers_the_forward_kernels():
    h = hashlib.sha256()
    for f in ("moe.hip", "gemv.hip", "e4b_device.h"):
        with open(os.path.join(ROOT, "bit_quantized_mixture_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    assert bench.kernel_source_sha() == h.hexdigest()[:16]


def test_committed_counters_match_the_committed_kernels():
    """The HBM traffic that bench.py reports comes from counters taken on these exact sources:
    every workload row of the counter table is keyed to the present hash, so the headline's
    `traffic` is not null."""
    for name in ("skewed_nf4_prefill", "mixtral_nf4_prefill", "mxfp4_moe", "finegrained_nf4_decode"):
        c = bench.load_counters(name)
        assert set(c) == {"gemm_gate_up", "gemm_down"}, name
        assert all(v > 0 for v in c.values())
    assert bench.load_counters("no_such_workload") == {}


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profile_summaries_name_the_present_kernel_sources():
    """Every committed trace/counter summary of the forward kernels states the hash of the
    sources it was taken on; it must be the present one."""
    sha = bench.kernel_source_sha()
    seen = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        with open(path) as f:
            text = f.read()
        for m in re.finditer(r"kernel sources sha ([0-9a-f]{16})", text):
            assert m.group(1) == sha, os.path.basename(path)
            seen += 1
    assert seen >= 6
