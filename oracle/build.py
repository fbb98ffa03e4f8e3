"""Compile the C oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(out: str = LIB, mutant: int = 0, quiet: bool = True) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
