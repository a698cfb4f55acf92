"""The oracle is test infrastructure and the product path has no fallback.

- Nothing in the package, and no csrc source, imports or names the oracle
  module; the oracle imports nothing from the package.
- Outside tests/, only smoke() in __graft_entry__.py and the CPU-baseline
  leg of bench.py import the oracle.
- Without the built library the binding raises instead of computing
  anything (there is no CPU path to fall back to).
"""
import ast
import glob
import os

import pytest

import recurrent_state_quant_amd as lq
from recurrent_state_quant_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "recurrent_state_quant_amd")


def _imports(path):
    """(module name, enclosing top-level function or None) of every import."""
    tree = ast.parse(open(path).read(), path)
    out = []
    for top in tree.body:
        fn = top.name if isinstance(top, (ast.FunctionDef, ast.AsyncFunctionDef)) else None
        for node in ast.walk(top):
            if isinstance(node, ast.Import):
                out += [(a.name, fn) for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                out.append((("." * node.level) + (node.module or ""), fn))
    return out


def test_package_does_not_use_the_oracle():
    files = glob.glob(os.path.join(PKG, "**", "*.py"), recursive=True)
    assert files
    for f in files:
        for mod, _ in _imports(f):
            assert not mod.split(".")[0] == "oracle", (f, mod)
    for f in glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")):
        assert "oracle" not in open(f, errors="replace").read().lower(), f


def test_oracle_does_not_use_the_package():
    files = glob.glob(os.path.join(ROOT, "oracle", "**", "*.py"), recursive=True)
    assert files
    for f in files:
        for mod, _ in _imports(f):
            assert not mod.startswith("recurrent_state_quant_amd") and not mod.startswith("tests"), (f, mod)


def test_oracle_imports_outside_tests():
    allowed = {os.path.join(ROOT, "__graft_entry__.py"): {"smoke"},
               # the CPU-baseline leg and its worker processes
               os.path.join(ROOT, "bench.py"): {"cpu_baseline", "_oracle_group"}}
    for f in glob.glob(os.path.join(ROOT, "*.py")):
        for mod, fn in _imports(f):
            if mod.split(".")[0] == "oracle":
                assert fn in allowed.get(f, set()), (f, mod, fn)


def test_binding_raises_without_the_library(monkeypatch):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", os.path.join(ROOT, "no-such-dir", "libleapquant.so"))
    with pytest.raises(ImportError):
        L.load()
    with pytest.raises(ImportError):
        lq.leapquant_abi_version()
