"""Host-side contract of the product path (no GPU needed): the library fails
loudly when missing, nothing in the package touches the oracle, and the bench
refuses GPU counts other than one before touching a device."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_missing_library_raises(tmp_path):
    from adaptive_head_budget_amd import lib
    saved = lib._lib
    lib._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            lib.load(str(tmp_path / "libadakv.so"))
    finally:
        lib._lib = saved


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom) and node.module:
            yield node.module


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "adaptive_head_budget_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                mods = list(_imports(os.path.join(dirpath, f)))
                assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (f, mods)


def test_bench_oracle_use_is_the_cpu_baseline_only():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.ImportFrom) and node.module and node.module.split(".")[0] == "oracle":
                    users.add(fn.name)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any(getattr(n, "module", None) == "oracle" or any(a.name.startswith("oracle") for a in n.names)
                   for n in top)
    assert users == {"cpu_baseline"}


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
