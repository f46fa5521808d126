"""Builds libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m exact_attention_60_amd._build``; the library lands next to
this file, in the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["api.cpp", "prefill.hip", "prefill_pipe.hip", "prefill_hd.hip", "prefill_d256.hip", "prefill_fp8.hip", "decode.hip", "decode_noalloc.hip", "backward.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    tmp = os.path.join(HERE, "_build")
    os.makedirs(tmp, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp, src + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage and src.endswith(".hip"):
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        if resource_usage:
            for line in r.stderr.splitlines():
                if "remark" in line and any(k in line for k in (
                        "Function Name", "VGPRs", "AGPRs", "Scratch", "Occupancy", "LDS")):
                    print(line.split("remark:")[-1].strip())
        objs.append(obj)
    tmp_lib = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", *objs, "-o", tmp_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--usage" in sys.argv))
