"""The oracle and the HIP path stay apart.

The oracle is test infrastructure: the package never imports or reads it,
the two share no source (the oracle includes only the C library, the HIP
sources only their own headers and HIP's), and bench.py touches it only in
its CPU-baseline function.  The seeded input generator, the one module both
sides use, holds no dispatch or combine arithmetic.  CPU only.
"""
import ast
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_get_dispatch_04_amd")
CSRC = os.path.join(PKG, "csrc")


def _files(d, exts):
    for base, _, names in os.walk(d):
        for n in names:
            if n.endswith(exts):
                yield os.path.join(base, n)


def test_package_never_names_the_oracle():
    for p in _files(PKG, (".py", ".hip", ".h", ".cpp", ".c")):
        text = open(p, encoding="utf-8").read()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), p
        assert "oracle/" not in text and "oracle.c" not in text, p


def test_no_shared_source():
    allowed_hip = {"ep.h", "ep_common.h", "ep_internal.h", "hip/hip_runtime.h", "algorithm",
                   "initializer_list", "stdint.h", "stddef.h", "atomic", "mutex"}
    for p in _files(CSRC, (".hip", ".h")):
        for inc in re.findall(r'^#include\s+[<"]([^>"]+)[>"]', open(p).read(), re.M):
            assert inc in allowed_hip, (p, inc)
    oracle_src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    for inc in re.findall(r'^#include\s+[<"]([^>"]+)[>"]', oracle_src, re.M):
        assert inc in {"math.h", "stdint.h", "stdlib.h", "string.h", "omp.h"}, inc


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    parents = {}
    for node in ast.walk(tree):
        for ch in ast.iter_child_nodes(node):
            parents[ch] = node
    found = []
    for node in ast.walk(tree):
        names = []
        if isinstance(node, ast.Import):
            names = [a.name for a in node.names]
        elif isinstance(node, ast.ImportFrom):
            names = [node.module or ""]
        if any(n == "oracle" or n.startswith("oracle.") for n in names):
            fn = node
            while fn in parents and not isinstance(fn, ast.FunctionDef):
                fn = parents[fn]
            found.append(getattr(fn, "name", "<module>"))
    assert found == ["cpu_baseline"], found


def test_importing_the_package_loads_no_oracle():
    code = ("import sys; import combine_get_dispatch_04_amd.api, combine_get_dispatch_04_amd._native, "
            "combine_get_dispatch_04_amd.workloads; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       check=True)
    assert r.stdout.strip() == "False"


def test_input_generator_has_no_path_arithmetic():
    """It draws inputs and names workloads (a quant mode is only a label
    there); it neither calls the library nor quantises, scatters or sums."""
    text = open(os.path.join(PKG, "workloads.py")).read()
    for word in ("libep", "_native", "ctypes", "ep_dispatch", "ep_combine", "448", "amax",
                 "e4m3_from", "float8"):
        assert word not in text, word
