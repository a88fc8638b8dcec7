"""Planted mistakes in the oracle must be caught by its pins.

Each mutant below is oracle/oracle.c with one plausible mistake (a dropped
term, a wrong constant, sign, index or operator, a transposed operand, a
reversed order), compiled to a scratch library and loaded by the pin tests
of the part it breaks (through ORACLE_LIB).  Every mutant must make those
tests fail; the unmutated source, compiled the same way, must pass them.
The mistakes stay inside the arrays' bounds, so a mutant fails by its
values, not by a crash.  Each one changes some result: a cap of 61440 on
E5M2, say, would not (rounding to two fraction bits leaves 57344 or 65536,
and both clamp to code 0x7B), so such equivalent mutants are left out.
CPU only.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

TC = "test_oracle_token_choice.py"
FMT = "test_oracle_formats.py"
QNT = "test_oracle_quant.py"
EC = "test_oracle_expert_choice.py"
RK = "test_oracle_ranks.py"

# (what, exact text in oracle.c, replacement, pin module that must catch it)
MUTANTS = [
    ("layout: rank of an expert taken modulo R",
     "row[e / per_rank] = 1;", "row[e % R] = 1;", TC),
    ("layout: tokens_per_rank counts every token",
     "tokens_per_rank[r] += row[r];", "tokens_per_rank[r] += 1;", TC),
    ("layout: invalid entries not counted",
     "            if (e < 0 || e >= E) {\n                (*num_invalid)++;\n                continue;\n            }\n            counts[e]++;",
     "            if (e < 0 || e >= E) {\n                continue;\n            }\n            counts[e]++;", TC),
    ("layout: -1 taken as invalid",
     "            if (e == -1)\n                continue;\n            if (e < 0 || e >= E) {\n                (*num_invalid)++;",
     "            if (e == -2)\n                continue;\n            if (e < 0 || e >= E) {\n                (*num_invalid)++;", TC),
    ("layout: offsets shifted by the expert's own count",
     "offsets[e + 1] = offsets[e] + counts[e];", "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);",
     TC),
    ("slots: k-major instead of token-major order",
     "    for (int t = 0; t < T; ++t) {\n        for (int k = 0; k < K; ++k) {\n            int64_t i = (int64_t)t * K + k;",
     "    for (int k = 0; k < K; ++k) {\n        for (int t = 0; t < T; ++t) {\n            int64_t i = (int64_t)t * K + k;",
     TC),
    ("slots: padded slot drops the rank",
     "(int64_t)e * cap_or_max_rows + r : -1;", "(int64_t)e * cap_or_max_rows : -1;", TC),
    ("slots: dropped slots not counted",
     "            if (s < 0) {\n                (*num_dropped)++;", "            if (s < 0) {\n", TC),
    ("bf16 dispatch: half of each row copied",
     "memcpy(recv + (int64_t)s * H, x + (int64_t)t * H, (size_t)H * sizeof(uint16_t));",
     "memcpy(recv + (int64_t)s * H, x + (int64_t)t * H, (size_t)H);", TC),
    ("fp8: scale divides by 447",
     "float sg = a / 448.0f;", "float sg = a / 447.0f;", TC),
    ("fp8: element multiplied by the scale",
     "oracle_e4m3_from_f32(v / sg);", "oracle_e4m3_from_f32(v * sg);", TC),
    ("fp8: group max without the absolute value",
     "float v = fabsf(oracle_bf16_to_f32(xr[128 * g + i]));",
     "float v = oracle_bf16_to_f32(xr[128 * g + i]);", TC),
    ("e4m3: subnormal boundary one binade low",
     "int qexp = (ex < -6) ? -9 : ex - 3;", "int qexp = (ex < -7) ? -10 : ex - 3;", FMT),
    ("e4m3: ties rounded away from zero",
     "double q = nearbyint(ldexp(a, -qexp));   /* RNE to an integer multiple of 2^qexp */",
     "double q = floor(ldexp(a, -qexp) + 0.5);", FMT),
    ("e4m3: sign of zero lost",
     "uint8_t sign = signbit(v) ? 0x80u : 0x00u;", "uint8_t sign = (v < 0) ? 0x80u : 0x00u;", FMT),
    ("bf16 rounding: ties away from zero",
     "double q = nearbyint(ldexp(a, -qexp));   /* exact scaling, then RNE */",
     "double q = floor(ldexp(a, -qexp) + 0.5);", FMT),
    ("per-token: int8 scale divides by 128",
     "const float Q = fmt == 1 ? 127.0f : 448.0f;", "const float Q = fmt == 1 ? 128.0f : 448.0f;",
     QNT),
    ("int8: clamped to -128",
     "    if (q < -127.0)\n        q = -127.0;", "    if (q < -128.0)\n        q = -128.0;", QNT),
    ("int8: ties rounded away from zero",
     "double q = nearbyint((double)v);", "double q = round((double)v);", QNT),
    ("per-token: max over the row without the absolute value",
     "float v = fabsf(oracle_bf16_to_f32(xr[i]));", "float v = oracle_bf16_to_f32(xr[i]);", QNT),
    ("MX: shared exponent off by one",
     "E = (e - 1) - emax;", "E = e - emax;", QNT),
    ("MX: e2m1 emax 3",
     "static const int emax_of[3] = {8, 15, 2};", "static const int emax_of[3] = {8, 15, 3};", QNT),
    ("MXFP4: nibbles swapped",
     "<< (4 * (c & 1))", "<< (4 * (1 - (c & 1)))", QNT),
    ("e5m2: saturates one code low, at 49152",
     "round_to_format(fabs((double)v), 2, -14, 57344.0)", "round_to_format(fabs((double)v), 2, -14, 49152.0)",
     QNT),
    ("e2m1: smallest normal exponent 1",
     "round_to_format(fabs((double)v), 1, 0, 6.0)", "round_to_format(fabs((double)v), 1, 1, 6.0)", QNT),
    ("combine: weights ignored",
     "double wk = w ? (double)w[(int64_t)t * K + k] : 1.0;", "double wk = 1.0;", TC),
    ("combine: weight index transposed",
     "double wk = w ? (double)w[(int64_t)t * K + k] : 1.0;",
     "double wk = w ? (double)w[(int64_t)k * T + t] : 1.0;", TC),
    ("expert choice: invalid entries not counted",
     "        if (i < 0 || i >= T) {\n            inval++;\n            continue;\n        }\n        memcpy(recv + j * H",
     "        if (i < 0 || i >= T) {\n            continue;\n        }\n        memcpy(recv + j * H", EC),
    ("expert choice: a token's entries in descending order",
     "    for (int64_t j = 0; j < n; ++j) {\n        int32_t i = token_indices[j];\n        if (i >= 0 && i < T)\n            tok_ent[",
     "    for (int64_t j = n - 1; j >= 0; --j) {\n        int32_t i = token_indices[j];\n        if (i >= 0 && i < T)\n            tok_ent[",
     EC),
    ("expert choice: combine weights ignored",
     "acc[h] += (double)w[j] * (double)oracle_bf16_to_f32(yr[h]);",
     "acc[h] += (double)oracle_bf16_to_f32(yr[h]);", EC),
    ("rank pack: rank of an expert taken modulo R",
     "if (e >= 0 && e < E && e / per_rank == r)\n                    on_rank = 1;",
     "if (e >= 0 && e < E && e % R == r)\n                    on_rank = 1;", RK),
    ("rank pack: local id not shifted",
     "send_idx[p * K + k] = here ? e - r * per_rank : -1;", "send_idx[p * K + k] = here ? e : -1;",
     RK),
    ("rank pack: other ranks' weights kept",
     "send_w[p * K + k] = here ? (w ? w[(int64_t)t * K + k] : 1.0f) : 0.0f;",
     "send_w[p * K + k] = w ? w[(int64_t)t * K + k] : 1.0f;", RK),
    ("rank pack: dropped rows not counted",
     "            if (p >= max_rows) {\n                (*num_dropped)++;",
     "            if (p >= max_rows) {\n", RK),
    ("partial combine: rounded to bf16 instead of fp32",
     "partial[(int64_t)p * H + h] = (float)acc[h];",
     "partial[(int64_t)p * H + h] = oracle_bf16_to_f32(oracle_bf16_from_f64(acc[h]));", RK),
    ("partial combine: weights ignored",
     "double wk = w ? (double)w[(int64_t)p * K + k] : 1.0;", "double wk = 1.0;", RK),
    ("rank sum: the last rank left out",
     "        for (int r = 0; r < R; ++r) {\n            int32_t p = pack_pos[(int64_t)t * R + r];",
     "        for (int r = 0; r + 1 < R; ++r) {\n            int32_t p = pack_pos[(int64_t)t * R + r];",
     RK),
]


def _build(src_text, d, name):
    c = os.path.join(d, name + ".c")
    so = os.path.join(d, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *CFLAGS, c, "-o", so, "-lm"], check=True, capture_output=True)
    return so


def _pins_pass(so, module):
    env = dict(os.environ, ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, module), "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode == 0


def test_mutations_are_exact_and_unique():
    src = open(SRC).read()
    for what, old, new, _ in MUTANTS:
        assert src.count(old) == 1, what
        assert old != new, what


@pytest.mark.slow
def test_planted_mistakes_are_caught():
    src = open(SRC).read()
    with tempfile.TemporaryDirectory() as d:
        clean = _build(src, d, "clean")
        for module in sorted({m for *_, m in MUTANTS}):
            assert _pins_pass(clean, module), f"the unmutated oracle fails {module}"

        def run(i):
            what, old, new, module = MUTANTS[i]
            so = _build(src.replace(old, new), d, f"mutant{i}")
            return what, _pins_pass(so, module)

        with ThreadPoolExecutor(6) as ex:
            results = list(ex.map(run, range(len(MUTANTS))))
    survivors = [what for what, passed in results if passed]
    assert not survivors, f"pins missed: {survivors}"
