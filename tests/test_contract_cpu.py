"""Host-side checks of how the pieces fit together (no GPU needed): the bench
refuses more than one GPU, the product path never reaches the oracle, and the
binding fails loudly instead of falling back when the HIP library is absent."""
from __future__ import annotations

import ast
import json
import os
import subprocess
import sys

import pytest

import sparse_mla_top_amd as smla
from sparse_mla_top_amd import build as smla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    msg = json.loads(res.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


@pytest.mark.parametrize("pkg", ["sparse_mla_top_amd", "workloads"])
def test_product_never_imports_the_oracle(pkg):
    for dirpath, _, files in os.walk(os.path.join(ROOT, pkg)):
        for f in files:
            if f.endswith(".py"):
                assert "oracle" not in _imports(os.path.join(dirpath, f)), os.path.join(dirpath, f)


def test_hip_library_built_from_its_own_sources_only():
    for src in smla_build.SOURCES + smla_build.HEADERS:
        path = os.path.normpath(os.path.join(smla_build.CSRC, src))
        assert not path.startswith(os.path.join(ROOT, "oracle")), src
        assert "oracle" not in open(path).read().lower(), src   # no shared code, not even by name


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(smla, "_lib", None)
    monkeypatch.setattr(smla, "LIB_PATH", os.path.join(ROOT, "no-such-dir", "libsparse_mla.so"))
    with pytest.raises(RuntimeError, match="missing"):
        smla.lib()
