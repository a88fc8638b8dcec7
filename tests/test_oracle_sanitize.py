"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_sanitize.c calls every oracle function on seeded
random and edge-case inputs, with each buffer allocated at exactly the size
its contract states.  Built with gcc's address, undefined and
float-cast-overflow sanitizers (and leak detection), the run must be clean.
To show the build would notice, two copies of oracle.c with a planted
mistake (a row copy one element too long, a buffer never freed) must each
be reported.  CPU only.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "sanitize", "oracle_sanitize.c")
ORACLE = os.path.join(ROOT, "oracle", "oracle.c")
FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
         "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]

PLANTED = {
    "overflow": ("memcpy(recv + (int64_t)s * H, x + (int64_t)t * H, (size_t)H * sizeof(uint16_t));",
                 "memcpy(recv + (int64_t)s * H, x + (int64_t)t * H, (size_t)(H + 1) * sizeof(uint16_t));",
                 "heap-buffer-overflow"),
    "leak": ("    free(cursor);\n}", "}", "detected memory leaks"),
}


def _run(src, d, name):
    exe = os.path.join(d, name)
    subprocess.run(["gcc", *FLAGS, DRIVER, src, "-o", exe, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.fixture(scope="module")
def workdir():
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_oracle_runs_clean_under_sanitizers(workdir):
    r = _run(ORACLE, workdir, "clean")
    assert r.returncode == 0, r.stderr[-3000:]
    assert "run clean" in r.stdout


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_sanitizer_build_reports_a_planted_mistake(workdir, name):
    old, new, report = PLANTED[name]
    src = open(ORACLE).read()
    assert src.count(old) >= 1
    p = os.path.join(workdir, f"planted_{name}.c")
    with open(p, "w") as f:
        f.write(src.replace(old, new, 1))
    r = _run(p, workdir, f"planted_{name}")
    assert r.returncode != 0
    assert report in r.stderr
