"""Runs host test modules against sanitizer builds of the library's host code
and of the C oracle (child process of tests/test_sanitize_host.py, started
with the AddressSanitizer runtime preloaded).

    python run_sanitized.py LIBMLA_SAN LIBORACLE_SAN TEST_FILE... [-k EXPR]
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import pytest  # noqa: E402


class UseSanitizedBuilds:
    def __init__(self, libmla, liboracle):
        self.libmla, self.liboracle = libmla, liboracle

    def pytest_configure(self, config):
        import paged_mla_decode_06_amd as mla
        import oracle
        mla.LIB_PATH = self.libmla
        mla._lib = None
        oracle._default = oracle.Oracle(self.liboracle)

    def pytest_sessionfinish(self, session, exitstatus):
        # the modules ran against the sanitizer builds, not the regular ones
        import paged_mla_decode_06_amd as mla
        import oracle
        assert mla._lib is not None and mla._lib._name == self.libmla, "the sanitized libmla was not loaded"
        assert oracle._default.path == self.liboracle, "the sanitized oracle was not loaded"


if __name__ == "__main__":
    libmla, liboracle = sys.argv[1], sys.argv[2]
    args = sys.argv[3:]
    sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu"] + args,
                         plugins=[UseSanitizedBuilds(libmla, liboracle)]))
