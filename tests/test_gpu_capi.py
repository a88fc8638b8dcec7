"""The C ABI from a plain C++ host program (tests/capi/roundtrip.cpp):
hipMalloc'd buffers, the entry points on the null stream, results checked
on the host by properties that hold at any size (counts and offsets, the
slot bijection and its order, received rows equal to their source rows, and
the exact unit-weight round trip bf16(m_t * x_t)), for token choice, the
one-launch low-latency dispatch, expert choice and one rank's share of the
exchange; the no-allocation call equal to the pair; and every round's layout
of a chunked prefill from one call, each round dispatched from its slice of
the workspace.  No Python between
the caller and libep."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "roundtrip")


def test_cpp_caller_round_trip():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    print("[case] C++ caller round trip", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi roundtrip ok" in r.stdout
