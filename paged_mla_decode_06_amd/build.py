"""Build libmla.so (gfx950 HIP kernels + host C ABI) in-tree with hipcc.

    python -m paged_mla_decode_06_amd.build [--resource-usage]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["mla_kernels.hip", "mla_append.hip", "mla_noalloc.hip", "mla_api.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC,
          # no packed fp32 instructions in any device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in VGPRs: the O accumulators are rescaled by VALU
          # code, which cannot touch AGPRs; the Q fragments (read-only MFMA
          # operands) then take the AGPRs
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wall", "-Wno-unused-function"]


def _run(cmd, quiet):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr)
    # the host pass does not know the device-only feature flag; harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    if out and not quiet:
        print(out, file=sys.stderr)
    return out


def build(out: str = LIB, quiet: bool = True, resource_usage: bool = False) -> str:
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage and src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        _run(cmd, quiet and not resource_usage)
        objs.append(obj)
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", out + ".tmp"], quiet)
    os.replace(out + ".tmp", out)
    for o in objs:
        os.remove(o)
    return out


if __name__ == "__main__":
    print(build(quiet=False, resource_usage="--resource-usage" in sys.argv))
