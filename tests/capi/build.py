"""Build tests/capi/roundtrip, a plain C++ host program that uses libep.so
through include/ep.h alone (run by tests/test_gpu_capi.py)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from combine_get_dispatch_04_amd import build as B  # noqa: E402

SRC = os.path.join(HERE, "roundtrip.cpp")
EXE = os.path.join(HERE, "roundtrip")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp"
    lib_dir = os.path.dirname(B.LIB)
    # the library is found next to the package, relative to this executable
    rpath = "$ORIGIN/" + os.path.relpath(lib_dir, HERE)
    cmd = [B.HIPCC, "-O2", "-std=c++17", "-Wall", f"-I{B.INCLUDE}", SRC, "-o", tmp,
           f"-L{lib_dir}", "-lep", f"-Wl,-rpath,{rpath}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
