"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/abi_host_sanitize.cpp drives every host path of libep that
runs without a GPU: the workspace sizing over a wide grid of shapes (T*K and
E*C up to just below 2^31) and the argument checks of the six entry points.
The library sources and the driver are built by hipcc with the sanitizers on
the host pass only (each -fsanitize= after -Xarch_host; the gfx950 code is
built as usual) and the run must be clean.  A copy of ep_api.hip that
computes T*K in 32-bit int must be reported, to show the build would notice
such a mistake.  CPU only (nothing here touches a GPU).
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
from combine_get_dispatch_04_amd import build as B  # noqa: E402

CSRC = os.path.join(ROOT, "combine_get_dispatch_04_amd", "csrc")
DRIVER = os.path.join(HERE, "sanitize", "abi_host_sanitize.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
FLAGS = [f for f in B.FLAGS if f not in ("-O3", "-shared", "-fPIC")] + ["-O1", "-g"] + SAN
INC = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
PLANT = ("    if ((int64_t)T * K > kI32)\n        return EP_ERR_INVALID_ARG;\n    return EP_OK;",
         "    if (T * K > kI32)\n        return EP_ERR_INVALID_ARG;\n    return EP_OK;")


def _compile(src, obj):
    subprocess.run([B.HIPCC, *FLAGS, *INC, "-c", src, "-o", obj], check=True, capture_output=True)


def _link_and_run(objs, exe):
    subprocess.run([B.HIPCC, *FLAGS, *objs, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.fixture(scope="module")
def objects():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not available")
    with tempfile.TemporaryDirectory() as d:
        objs = {}
        for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [DRIVER]:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            _compile(src, obj)
            objs[os.path.basename(src)] = obj
        yield d, objs


def test_abi_host_code_runs_clean(objects):
    d, objs = objects
    r = _link_and_run(list(objs.values()), os.path.join(d, "clean"))
    assert r.returncode == 0, r.stderr[-3000:]
    assert "run clean" in r.stdout


def test_planted_int_overflow_is_reported(objects):
    d, objs = objects
    src = open(os.path.join(CSRC, "ep_api.hip")).read()
    assert src.count(PLANT[0]) == 1
    planted = os.path.join(d, "ep_api_planted.hip")
    with open(planted, "w") as f:
        f.write(src.replace(PLANT[0], PLANT[1]))
    obj = os.path.join(d, "ep_api_planted.o")
    _compile(planted, obj)
    r = _link_and_run([obj if k == "ep_api.hip" else v for k, v in objs.items()],
                      os.path.join(d, "planted"))
    assert r.returncode != 0
    assert "signed integer overflow" in r.stderr
