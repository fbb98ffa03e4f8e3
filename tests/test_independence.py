"""The oracle and the GPU path share no code, and the product path has no
CPU fallback (CPU only, reads the sources).

- Nothing in the package (Python binding, HIP kernels, host C++) names the
  oracle; nothing in the oracle names the package or its kernel sources.
- The seeded input generator imports neither side.
- bench.py reaches the oracle only inside its CPU-baseline function.
- Without the built library the binding raises instead of computing."""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_mla_decode_06_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    out = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out += [a.name.split(".")[0] for a in node.names]
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            out.append(node.module.split(".")[0])
    return out


def test_package_never_names_the_oracle():
    for f in _files(PKG, (".py", ".hip", ".cpp", ".h")):
        text = open(f).read()
        if f.endswith(".py"):
            assert "oracle" not in _imports(f), f"{f} imports the oracle"
        assert not re.search(r'#include\s+"[^"]*oracle', text), f"{f} includes an oracle header"
        assert "liboracle" not in text, f"{f} loads the oracle library"


def test_oracle_never_names_the_package():
    for f in _files(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        text = open(f).read()
        assert "paged_mla_decode_06_amd" not in text, f"{f} names the GPU package"
        assert "csrc" not in text and "libmla" not in text, f"{f} names the GPU sources or library"
        assert not re.search(r'#include\s+"mla_', text), f"{f} includes a kernel header"


def test_generator_imports_neither_side():
    for f in _files(os.path.join(ROOT, "mla_synth"), (".py",)):
        imps = _imports(f)
        assert "oracle" not in imps and "paged_mla_decode_06_amd" not in imps, f"{f} imports {imps}"


def test_bench_reaches_the_oracle_only_for_its_cpu_baseline():
    path = os.path.join(ROOT, "bench.py")
    tree = ast.parse(open(path).read())
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    for n in top:
        names = [a.name for a in n.names] if isinstance(n, ast.Import) else [n.module or ""]
        assert not any(x.split(".")[0] == "oracle" for x in names), "bench.py imports the oracle at module level"
    users = set()
    for fn in [n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)]:
        for node in ast.walk(fn):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                if any(m.split(".")[0] == "oracle" for m in mods):
                    users.add(fn.name)
    assert users == {"cpu_baseline"}, users


def test_missing_library_raises(monkeypatch):
    import paged_mla_decode_06_amd as mla
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libmla.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mla.lib()
    with pytest.raises(RuntimeError, match="not built"):
        mla.mla_abi_version()
