"""Host-side guards on the product path: it never reaches the CPU oracle,
it fails loudly when the HIP library is missing, and the benchmark refuses a
multi-GPU request (one GPU is all it measures)."""

from __future__ import annotations

import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_scaled_fp8_linear_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_package_never_imports_the_oracle_or_workloads():
    for name in os.listdir(PKG):
        if name.endswith(".py"):
            mods = list(_imports(os.path.join(PKG, name)))
            assert not any(m.split(".")[0] in ("oracle", "workloads") for m in mods), (name, mods)


def test_csrc_has_no_reference_to_the_oracle():
    csrc = os.path.join(PKG, "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name), errors="ignore").read().lower()
        assert "oracle" not in text, name


def test_missing_library_raises(monkeypatch):
    from block_scaled_fp8_linear_amd import _lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", os.path.join(PKG, "no_such_library.so"))
    with pytest.raises(ImportError):
        L.load()
    with pytest.raises(ImportError):
        L.workspace_size(4, 8, 16)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
