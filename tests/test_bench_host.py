"""Host logic of bench.py, on the CPU: the one-GPU guard, the --graph check,
the argument binding of the entry points, the configuration
keys, the bookkeeping that ties a committed profile to the kernel sources it
was taken on, and the checks the bench applies to its timed outputs (bit
for bit, and the NaN-proof combine tolerance)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("args", [["--steps", "25", "--graph", "10"], ["--graph", "-1"]])
def test_graph_steps_must_divide_the_timed_steps(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "multiple of --graph" in r.stderr
    assert r.stdout == ""


def test_bind_takes_addresses_once():
    class Buf:
        calls = 0

        def data_ptr(self):
            Buf.calls += 1
            return 4096

    seen = []
    f = bench.bind(lambda *a: seen.append(a), Buf(), 7, None, Buf())
    assert Buf.calls == 2
    f()
    f()
    assert Buf.calls == 2
    assert seen == [(4096, 7, None, 4096)] * 2


def test_bind_keeps_its_tensors_alive():
    """A buffer that only a bound call uses stays allocated while the call
    exists: with addresses alone, such a tensor was freed as soon as the
    step was built."""
    import gc
    import weakref

    import torch
    t = torch.empty(16, dtype=torch.int32)
    ref = weakref.ref(t)
    f = bench.bind(lambda *a: None, t, 3)
    del t
    gc.collect()
    assert ref() is not None
    del f
    gc.collect()
    assert ref() is None


def test_code_only_drops_comments_and_whitespace_only():
    a = "int x = 1; // one\n/* two\n lines */ int  y=2;\n"
    b = "int x = 1;\nint y=2;"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("a + b;") != bench._code_only("a - b;")
    # a comment marker inside a string literal is code
    assert "//x" in bench._code_only('const char *s = "//x"; // y')
    assert "y" not in bench._code_only('const char *s = "//x"; // y').split('"')[-1]


def test_kernel_source_hash_is_per_kernel_and_stable():
    comb = bench.kernel_source_hash("combine_kernel")
    disp = bench.kernel_source_hash("dispatch_kernel")
    whole = bench.kernel_source_hash(None)
    assert len({comb, disp, whole}) == 3
    assert bench.kernel_source_hash("combine_kernel") == comb
    # kernels built from the same files share a hash; an unlisted kernel
    # depends on every source
    assert bench.kernel_source_hash("partial_kernel") == comb
    assert bench.kernel_source_hash("no_such_kernel") == whole
    for h in (comb, disp, whole):
        assert len(h) == 64 and int(h, 16) >= 0


def test_profile_entries_follow_the_kernel_sources(monkeypatch):
    key = "prefill_T4096_H7168_E256_K8"
    # the headline's committed trace and counters were taken on these sources
    for kernel in ("dispatch_kernel", "combine_kernel"):
        assert bench.trace_avg_us(key, kernel) > 0
        assert bench.traffic_entry(key, kernel) > 0
    assert bench.trace_avg_us("no_such_configuration", "combine_kernel") is None
    assert bench.trace_avg_us(key, "no_such_kernel") is None
    # any other sources: the entries no longer apply
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel=None: "0" * 64)
    assert bench.trace_avg_us(key, "combine_kernel") is None
    assert bench.traffic_entry(key, "combine_kernel") is None


class _W:
    name = "prefill_T4096_H7168_E256_K8"
    default_quant = "bf16"


@pytest.mark.parametrize("meta,chunk,two_call,ranks,suffix", [
    ({"quant": "bf16"}, 0, False, 0, ""),
    ({}, 0, False, 0, ""),
    ({"quant": "fp8_e4m3_g128"}, 0, False, 0, "_fp8_e4m3_g128"),
    ({"quant": "bf16"}, 1024, False, 0, "_chunk1024"),
    ({"quant": "bf16"}, 0, True, 0, "_two_call"),
    ({"quant": "bf16"}, 0, False, 8, "_ranks8"),
    ({"quant": "mxfp4_e2m1"}, 512, False, 0, "_mxfp4_e2m1_chunk512"),
])
def test_workload_key(meta, chunk, two_call, ranks, suffix):
    assert bench.workload_key(_W, meta, chunk, two_call, ranks) == _W.name + suffix


def test_every_committed_profile_names_a_bench_configuration():
    """Each profiles/<kind>_<key>.json pairs with its other kind and carries a
    per-kernel source hash and the command that made it."""
    import json
    d = os.path.join(ROOT, "profiles")
    keys = {}
    for f in sorted(os.listdir(d)):
        if not f.endswith(".json"):
            continue
        kind, key = f[:-5].split("_", 1)
        keys.setdefault(key, set()).add(kind)
        with open(os.path.join(d, f)) as fh:
            t = json.load(fh)
        assert t.get("command") or t.get("commands"), f
        assert t.get("kernels"), f
        for name, k in t["kernels"].items():
            assert len(k.get("src_sha256", "")) == 64, (f, name)
    assert keys, "no profiles"
    for key, kinds in keys.items():
        assert kinds == {"kernels", "traffic"}, key


BF = {1.0: 0x3F80, 2.0: 0x4000, 0.0: 0x0000, -3.0: 0xC040}


def test_combine_check_is_nan_proof():
    ref = np.array([BF[1.0], BF[2.0], BF[0.0], BF[-3.0]], np.uint16)
    assert bench._combine_bad(ref, ref) == 0
    for bad in (0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80):     # NaN, -NaN, sNaN, +Inf, -Inf
        g = ref.copy()
        g[1] = bad
        assert bench._combine_bad(g, ref) == 1, hex(bad)
        assert bench._combine_bad(ref, g) == 1, hex(bad)      # a non-finite reference too


def test_combine_check_bound():
    # at 2.0 the bound is 2^-7 * 2 + 1e-3 = 0.016625: one bf16 ulp (2^-6) is
    # inside, two are outside
    ref = np.array([BF[2.0]], np.uint16)
    assert bench._combine_bad(np.array([0x4001], np.uint16), ref) == 0
    assert bench._combine_bad(np.array([0x4002], np.uint16), ref) == 1
    # near zero the absolute term decides: 2^-10 passes, 2^-9 does not
    z = np.array([BF[0.0]], np.uint16)
    assert bench._combine_bad(np.array([0x3A80], np.uint16), z) == 0     # 2^-10
    assert bench._combine_bad(np.array([0x3B00], np.uint16), z) == 1     # 2^-9


def test_f32_check():
    r = np.array([1.0, -2.0, 0.0], np.float32)
    assert bench._combine_bad_f32(r, r) == 0
    g = r.copy()
    g[0] = np.float32(1.0 + 2.0 ** -8)
    assert bench._combine_bad_f32(g, r) == 0
    g[0] = np.float32(1.0 + 2.0 ** -6)
    assert bench._combine_bad_f32(g, r) == 1
    for bad in (np.nan, np.inf, -np.inf):
        g = r.copy()
        g[2] = bad
        assert bench._combine_bad_f32(g, r) == 1


def test_checks_record_each_output():
    ck = bench._Checks()
    a = np.arange(6, dtype=np.int32)
    ck.equal("same", a, a.copy())
    b = a.copy()
    b[3] = -1
    ck.equal("differs", b, a)
    ck.equal("shape", a[:5], a)
    # -0.0 and +0.0 differ bit for bit
    ck.equal("zero sign", np.array([-0.0], np.float32), np.array([0.0], np.float32))
    ck.close("combine", np.array([0x4001], np.uint16), np.array([0x4000], np.uint16))
    ck.close("combine nan", np.array([0x7FC0], np.uint16), np.array([0x4000], np.uint16))
    assert ck.done == ["same", "combine"]
    assert ck.failed == ["differs", "shape", "zero sign", "combine nan (1)"]


def test_frac_by_trace():
    assert bench.frac_by_trace(8e12 * 90e-6, 90.0) == pytest.approx(1.0)
    assert bench.frac_by_trace(528744448, 90.33) == pytest.approx(0.7317, abs=1e-4)
    assert bench.frac_by_trace(1.0, None) is None
