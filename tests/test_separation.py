"""The product path and the oracle are kept apart.

The oracle (oracle/) is test infrastructure: only the tests, the smoke check and the benchmark's
CPU baseline use it, and it shares no code with the HIP path.  The seeded input generators
(workloads/) serve both sides and import neither.  These checks read the sources and the built
library's dynamic section, and import the package in a fresh process; they need no GPU.
"""
import ast
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_compression_tensor_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _sources(d, exts):
    for dirpath, dirnames, files in os.walk(d):
        dirnames[:] = [x for x in dirnames if x != "__pycache__"]
        for f in sorted(files):
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def _imported_modules(path):
    """(module name, enclosing top-level function or None) of every import in a Python file."""
    tree = ast.parse(open(path).read())
    out = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = func
            if func is None and isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)):
                f = child.name
            if isinstance(child, ast.Import):
                out.extend((a.name, f) for a in child.names)
            elif isinstance(child, ast.ImportFrom) and child.level == 0:
                out.append((child.module or "", f))
            visit(child, f)

    visit(tree, None)
    return out


def test_product_sources_never_name_the_oracle():
    files = list(_sources(PKG, (".py", ".hip", ".hpp", ".cpp", ".h")))
    files.append(os.path.join(ROOT, "include", "tfp8.h"))
    assert len(files) >= 5
    for f in files:
        assert not re.search(r"oracle", open(f).read(), re.IGNORECASE), f


def test_oracle_sources_never_name_the_product():
    files = list(_sources(ORACLE, (".py", ".c", ".h")))
    assert len(files) >= 4
    for f in files:
        text = open(f).read()
        for name in ("fp8_compression_tensor_amd", "tfp8_kernels", "tfp8_device", "tfp8.h",
                     "libtfp8.so", "hip"):
            assert not re.search(r"\b" + re.escape(name), text), (f, name)


def test_shared_input_generators_import_neither_side():
    for f in _sources(os.path.join(ROOT, "workloads"), (".py",)):
        for mod, _ in _imported_modules(f):
            top = mod.split(".")[0]
            assert top not in ("oracle", "fp8_compression_tensor_amd", "torch"), (f, mod)


def test_bench_uses_the_oracle_only_in_its_cpu_baseline():
    uses = [(m, f) for m, f in _imported_modules(os.path.join(ROOT, "bench.py"))
            if m.split(".")[0] == "oracle"]
    assert uses and all(f == "cpu_baseline" for _, f in uses), uses


def test_graft_entry_uses_the_oracle_only_to_build_it_and_in_smoke():
    uses = [(m, f) for m, f in _imported_modules(os.path.join(ROOT, "__graft_entry__.py"))
            if m.split(".")[0] == "oracle"]
    assert uses and all(f in ("build", "smoke") for _, f in uses), uses


def test_library_links_no_oracle():
    lib = os.path.join(PKG, "libtfp8.so")
    if not os.path.exists(lib):
        pytest.skip("library not built")
    dyn = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[(.+?)\]", dyn)
    assert needed and not any("oracle" in n for n in needed), needed
    syms = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True,
                          check=True).stdout
    assert "tfp8_compress" in syms and "tfp8_ref_" not in syms


def test_importing_the_package_loads_no_oracle():
    code = ("import sys, fp8_compression_tensor_amd\n"
            "bad = [k for k in sys.modules if k.split('.')[0] in ('oracle', 'workloads')]\n"
            "assert not bad, bad\n")
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True, timeout=600)


def test_missing_library_fails_loudly(monkeypatch):
    import fp8_compression_tensor_amd as m

    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libtfp8.so"))
    with pytest.raises(RuntimeError, match="not built"):
        m.lib()
