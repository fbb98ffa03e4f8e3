"""The host code of the library (argument checks, workspace layout, the
planner's host mirror in mla_plan.h, mla_plan_host, mla_check_inputs_host,
mla_check_qo_indptr_host) and the C oracle, built with g++/gcc under
AddressSanitizer and UndefinedBehaviorSanitizer, run through the host test
modules' plan, validation and oracle-pin cases: every case must pass with no
sanitizer report (any report aborts the child process).  The device side is
replaced by stand-ins that report "no device" (tests/sanitize/host_stubs.cpp)."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_mla_decode_06_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]
    return r


def test_host_code_and_oracle_under_sanitizers(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime for gcc")
    libmla = str(tmp_path / "libmla_san.so")
    liboracle = str(tmp_path / "liboracle_san.so")
    _run(["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN +
         [os.path.join(CSRC, "mla_api.cpp"), os.path.join(HERE, "sanitize", "host_stubs.cpp"), "-o", libmla])
    _run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp"] + SAN +
         [os.path.join(ROOT, "oracle", "oracle.c"), "-o", liboracle, "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "run_sanitized.py"), libmla, liboracle,
                        os.path.join(HERE, "test_plan.py"), os.path.join(HERE, "test_abi_host.py"),
                        os.path.join(HERE, "test_oracle.py"), os.path.join(HERE, "test_oracle_ragged.py")],
                       capture_output=True, text=True, env=env, cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out, out[-2000:]
