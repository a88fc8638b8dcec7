"""Build tests/hwcheck/libconvert_check.so, the test-only library that checks
the dispatch kernel's element arithmetic exhaustively on the GPU."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from combine_get_dispatch_04_amd import build as B  # noqa: E402

SRC = os.path.join(HERE, "convert_check.hip")
LIB = os.path.join(HERE, "libconvert_check.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [B.HIPCC, *B.FLAGS, f"-I{B.CSRC}", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
