"""Build the e4b HIP library (libe4b.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libe4b.so")
SOURCES = ["abi.hip", "pack.hip", "route.hip", "moe.hip", "gemv.hip", "dgrad.hip", "int4.hip", "probe.hip", "scaled.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the e4b library)")


def compile_cmd(out: str) -> list[str]:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # correctly rounded float32 division (the NF4 packer divides by absmax) and no
        # value-changing fast-math
        "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
        # keep the compiler from forming packed-fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument", "-I" + INCLUDE,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def resource_usage(source: str) -> dict[str, dict[str, int]]:
    """Register use of every kernel of one source file, as the compiler reports it
    (-Rpass-analysis=kernel-resource-usage on a device-only compile): mangled kernel name ->
    {"vgpr", "agpr", "vgpr_spill", "scratch", "occupancy"}."""
    import re
    import tempfile

    flags = compile_cmd("x")[1:]
    flags = [f for f in flags if f not in ("-shared", "-o", "x") and not f.endswith(".hip")]
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hipcc(), *flags, "--cuda-device-only", "-c", os.path.join(CSRC, source),
               "-o", os.path.join(tmp, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "VGPRs Spill": "vgpr_spill",
            "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy"}
    out: dict[str, dict[str, int]] = {}
    cur = None
    for ln in r.stderr.splitlines():
        m = re.search(r"remark:\s+(Function Name|[A-Za-z][A-Za-z /\[\]]*?): (\S+)", ln)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in keys:
            cur[keys[key]] = int(val)
    return out


def build(verbose: bool = False, out: str = LIB) -> str:
    """Compile every source to an object in parallel (one hipcc per source), then link the
    shared library; the result replaces `out` only when every step succeeded."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    flags = [f for f in compile_cmd("x")[1:] if f not in ("-shared", "-o", "x") and not f.endswith(".hip")]
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    noise = "is not a recognized feature for this target"

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
        return r.returncode, msgs

    with tempfile.TemporaryDirectory() as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[hipcc(), *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
            results = list(ex.map(run, cmds))
        for rc, msgs in results:
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
            if verbose and msgs:
                print("\n".join(msgs), file=sys.stderr)
        tmp_out = out + ".tmp"
        rc, msgs = run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_out])
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
