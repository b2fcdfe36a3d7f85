"""The product path and the oracle share no code.

The package (its Python modules and every HIP/C++ source and header) never
imports, includes or names the oracle package, and the oracle never imports
the package.  Only the seeded input generators (synthetic.py, which holds
none of the method's arithmetic) may be used by both sides, and the oracle
does not need even those.  bench.py (its CPU-baseline leg) and the smoke
entry point are the only files outside tests/ that call the oracle."""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_39_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _py_imports(path):
    tree = ast.parse(open(path).read(), path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            mods.add(node.module.split(".")[0])
        elif isinstance(node, ast.ImportFrom) and node.level > 0:
            mods.add("<relative>")
    return mods


def _files(top, exts):
    for d, _, fs in os.walk(top):
        if "__pycache__" in d:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_package_does_not_use_the_oracle():
    for path in _files(PKG, (".py",)):
        assert "oracle" not in _py_imports(path), path
    for path in _files(PKG, (".hip", ".cpp", ".h")):
        src = open(path).read()
        assert not re.search(r'#\s*include\s*[<"][^>"]*oracle', src), path


def test_oracle_does_not_use_the_package():
    for path in _files(ORACLE, (".py",)):
        mods = _py_imports(path)
        assert "mixture_experts_layer_39_amd" not in mods, path


def test_only_bench_and_smoke_call_the_oracle_outside_tests():
    users = []
    for name in os.listdir(ROOT):
        path = os.path.join(ROOT, name)
        if name.endswith(".py") and os.path.isfile(path) and "oracle" in _py_imports(path):
            users.append(name)
    assert sorted(users) == ["__graft_entry__.py", "bench.py"], users
