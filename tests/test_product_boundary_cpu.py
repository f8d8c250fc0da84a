"""The library path stands alone: it fails loudly without its HIP build and
never reaches the float64 oracle, which is test infrastructure only."""

import ast
import os
import re

import pytest

import sparse_attention_long_03_amd.binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_long_03_amd")


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libdsa.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def _imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield ("." * node.level) + (node.module or "")


def test_package_never_imports_the_oracle():
    seen = 0
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith(".py"):
                seen += 1
                for mod in _imported_modules(os.path.join(dirpath, f)):
                    assert "oracle" not in mod, f"{f} imports {mod}"
    assert seen > 0


def test_kernels_include_nothing_from_the_oracle():
    inc = re.compile(r'^\s*#\s*include\s*[<"]([^>"]+)[>"]', re.M)
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        for name in inc.findall(open(os.path.join(csrc, f)).read()):
            assert "oracle" not in name, f"{f} includes {name}"
