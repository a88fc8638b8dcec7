"""C-ABI checks that need no GPU: every symbol declared in include/ep.h is
exported by libep.so with the binding's arity; workspace sizing; and every
argument error is returned synchronously, before any launch.

Pointers below are fake, aligned addresses: every call here is rejected by
the host-side checks, so nothing is dereferenced or launched."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_get_dispatch_04_amd._native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(ep_\w+)\s*\(([^;{]*?)\)\s*;", src):
        args = [a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        out[m.group(1)] = len(args)
    return out


def test_header_declares_the_operations():
    d = _declared()
    for name in ("ep_get_dispatch_layout", "ep_dispatch", "ep_low_latency_dispatch",
                 "ep_combine", "ep_dispatch_expert_choice", "ep_combine_expert_choice"):
        assert name in d


def test_every_declared_symbol_is_exported_with_binding_arity():
    L = N.lib()
    d = _declared()
    assert set(d) == set(N.SIGNATURES)
    for name, nargs in d.items():
        assert hasattr(L, name), name
        assert len(N.SIGNATURES[name][1]) == nargs, name
    syms = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in syms.splitlines() if " T " in ln}
    assert set(d) <= exported


def test_status_strings():
    for s in range(5):
        assert N.status_string(s)
    assert N.status_string(0) == "ok"


def test_workspace_sizes():
    a = N.ep_workspace_bytes(4096, 8, 256, 1)
    assert a > 4096 * 8 * 4 and a % 256 == 0
    assert N.ep_workspace_bytes(4096, 8, 256, 8) >= a
    assert N.ep_workspace_bytes(0, 8, 256, 1) > 0
    assert N.ep_workspace_bytes(10, 0, 4, 1) == 0           # K < 1
    assert N.ep_workspace_bytes(10, 2, 6, 4) == 0           # E % R != 0
    assert N.ep_workspace_bytes(10, 2, 5000, 1) == 0        # E too large
    assert N.ep_workspace_bytes(-1, 2, 4, 1) == 0
    assert N.ep_workspace_bytes(3, 40000, 256, 16) >= 3 * 40000 * 4   # rows longer than a chunk
    assert N.ep_workspace_bytes(1, (1 << 31) - 1, 8, 1) > 0             # T*K just below 2^31
    assert N.ep_workspace_bytes(2, 1 << 30, 8, 1) == 0                 # T*K = 2^31
    assert N.ep_ec_workspace_bytes(8192, 64, 256) >= 64 * 256 * 4 + 8193 * 8
    assert N.ep_ec_workspace_bytes(8, 0, 4) == 0


A = 0x10000        # fake 256-aligned device address
B = 0x20000
WS = 0x100000


def _layout(**kw):
    args = dict(topk_idx=A, T=16, K=2, E=8, R=1, counts=A, offsets=A, tokens_per_rank=A,
                is_token_in_rank=A, num_invalid=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return N.ep_get_dispatch_layout(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(T=-1), N.EP_ERR_INVALID_ARG),
    (dict(E=0), N.EP_ERR_INVALID_ARG),
    (dict(E=4097), N.EP_ERR_UNSUPPORTED),
    (dict(E=8, R=3), N.EP_ERR_INVALID_ARG),
    (dict(R=2048, E=2048), N.EP_ERR_UNSUPPORTED),
    (dict(counts=None), N.EP_ERR_INVALID_ARG),
    (dict(offsets=None), N.EP_ERR_INVALID_ARG),
    (dict(num_invalid=None), N.EP_ERR_INVALID_ARG),
    (dict(topk_idx=None), N.EP_ERR_INVALID_ARG),
    (dict(topk_idx=A + 2), N.EP_ERR_INVALID_ARG),
    (dict(ws=None), N.EP_ERR_WORKSPACE),
    (dict(ws=WS + 16), N.EP_ERR_WORKSPACE),
    (dict(ws_bytes=16), N.EP_ERR_WORKSPACE),
    (dict(T=1 << 30, K=4), N.EP_ERR_INVALID_ARG),
])
def test_layout_rejects(kw, status):
    assert _layout(**kw) == status


def _layout_rounds(**kw):
    args = dict(topk_idx=A, T=16, K=2, E=8, R=1, round_tokens=4, counts=A, offsets=A,
                tokens_per_rank=A, is_token_in_rank=A, num_invalid=A, ws=WS, ws_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return N.ep_get_dispatch_layout_rounds(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(round_tokens=0), N.EP_ERR_INVALID_ARG),
    (dict(round_tokens=-3), N.EP_ERR_INVALID_ARG),
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(T=-1), N.EP_ERR_INVALID_ARG),
    (dict(E=4097), N.EP_ERR_UNSUPPORTED),
    (dict(E=8, R=3), N.EP_ERR_INVALID_ARG),
    (dict(counts=None), N.EP_ERR_INVALID_ARG),
    (dict(offsets=None), N.EP_ERR_INVALID_ARG),
    (dict(num_invalid=None), N.EP_ERR_INVALID_ARG),
    (dict(topk_idx=None), N.EP_ERR_INVALID_ARG),
    (dict(tokens_per_rank=A + 2), N.EP_ERR_INVALID_ARG),
    (dict(ws=None), N.EP_ERR_WORKSPACE),
    (dict(ws=WS + 16), N.EP_ERR_WORKSPACE),
    (dict(ws_bytes=16), N.EP_ERR_WORKSPACE),
])
def test_layout_rounds_rejects(kw, status):
    assert _layout_rounds(**kw) == status


def test_layout_rounds_workspace_bytes():
    """Full rounds of round_tokens, each the single-call workspace, then the
    shorter last round's; round_tokens >= T is one round."""
    one = N.ep_workspace_bytes
    for T, K, E, R, rt in [(4096, 8, 256, 1, 1024), (4100, 8, 256, 8, 1024), (10, 3, 16, 4, 3),
                           (7, 2, 8, 1, 100), (5, 1, 4, 1, 1), (100000, 8, 64, 1, 3000)]:
        full, last = divmod(T, min(rt, T))
        want = full * one(min(rt, T), K, E, R) + (one(last, K, E, R) if last else 0)
        assert N.ep_workspace_bytes_rounds(T, K, E, R, rt) == want, (T, K, E, R, rt)
    assert N.ep_workspace_bytes_rounds(0, 8, 256, 1, 64) == one(0, 8, 256, 1)
    assert N.ep_workspace_bytes_rounds(10, 2, 8, 1, 0) == 0
    assert N.ep_workspace_bytes_rounds(10, 0, 8, 1, 4) == 0
    assert N.ep_workspace_bytes_rounds(10, 2, 6, 4, 4) == 0


def _dispatch(**kw):
    args = dict(x=A, T=16, H=256, topk_idx=A, K=2, E=8, offsets=A, layout=0, cap_or_max_rows=32,
                quant=0, recv_x=B, recv_scales=None, slot=A, recv_src=A, num_dropped=A, ws=WS,
                ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return N.ep_dispatch(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(H=12), N.EP_ERR_INVALID_ARG),
    (dict(H=0), N.EP_ERR_INVALID_ARG),
    (dict(quant=1, H=200, recv_scales=A), N.EP_ERR_INVALID_ARG),     # fp8 needs H % 128 == 0
    (dict(quant=1, recv_scales=None), N.EP_ERR_INVALID_ARG),
    (dict(quant=7), N.EP_ERR_INVALID_ARG),
    (dict(quant=-1), N.EP_ERR_INVALID_ARG),
    (dict(quant=4, H=200, recv_scales=A), N.EP_ERR_INVALID_ARG),     # MX needs H % 32 == 0
    (dict(quant=6, H=48, recv_scales=A), N.EP_ERR_INVALID_ARG),
    (dict(quant=5, recv_scales=None), N.EP_ERR_INVALID_ARG),
    (dict(quant=3, recv_scales=None), N.EP_ERR_INVALID_ARG),
    (dict(quant=2, recv_scales=A + 2), N.EP_ERR_INVALID_ARG),       # fp32 scales: 4-byte alignment
    (dict(layout=5), N.EP_ERR_INVALID_ARG),
    (dict(cap_or_max_rows=-1), N.EP_ERR_INVALID_ARG),
    (dict(layout=1, E=4096, cap_or_max_rows=1 << 20), N.EP_ERR_INVALID_ARG),   # E*cap >= 2^31
    (dict(x=A + 8), N.EP_ERR_INVALID_ARG),                          # 16-byte alignment
    (dict(recv_x=B + 4), N.EP_ERR_INVALID_ARG),
    (dict(x=None), N.EP_ERR_INVALID_ARG),
    (dict(recv_x=None), N.EP_ERR_INVALID_ARG),
    (dict(slot=None), N.EP_ERR_INVALID_ARG),
    (dict(offsets=None), N.EP_ERR_INVALID_ARG),
    (dict(num_dropped=None), N.EP_ERR_INVALID_ARG),
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(E=9000), N.EP_ERR_UNSUPPORTED),
    (dict(H=(1 << 24) + 8), N.EP_ERR_UNSUPPORTED),                   # row bytes stay 32-bit
    (dict(ws=None), N.EP_ERR_WORKSPACE),
    (dict(ws_bytes=100), N.EP_ERR_WORKSPACE),
])
def test_dispatch_rejects(kw, status):
    assert _dispatch(**kw) == status


def _noalloc(**kw):
    args = dict(x=A, T=16, H=256, topk_idx=A, K=2, E=8, R=1, counts=A, offsets=A,
                tokens_per_rank=A, is_token_in_rank=A, num_invalid=A, layout=0,
                cap_or_max_rows=32, quant=0, recv_x=B, recv_scales=None, slot=A, recv_src=A,
                num_dropped=A, stream=None)
    args.update(kw)
    return N.ep_layout_dispatch_noalloc(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(E=8, R=3), N.EP_ERR_INVALID_ARG),
    (dict(R=2048, E=2048), N.EP_ERR_UNSUPPORTED),
    (dict(counts=None), N.EP_ERR_INVALID_ARG),
    (dict(num_invalid=A + 2), N.EP_ERR_INVALID_ARG),
    (dict(H=12), N.EP_ERR_INVALID_ARG),
    (dict(quant=1, recv_scales=None), N.EP_ERR_INVALID_ARG),
    (dict(layout=5), N.EP_ERR_INVALID_ARG),
    (dict(x=A + 8), N.EP_ERR_INVALID_ARG),
    (dict(slot=None), N.EP_ERR_INVALID_ARG),
    # tables beyond the library's scratch array (8 MiB): use the pair instead
    (dict(T=1 << 20, K=4, cap_or_max_rows=1 << 22), N.EP_ERR_UNSUPPORTED),
    (dict(T=600000, K=4, cap_or_max_rows=2400000), N.EP_ERR_UNSUPPORTED),
])
def test_noalloc_rejects(kw, status):
    """Rejected on the host before anything is enqueued, like the pair;
    sizes whose tables exceed the scratch array are refused."""
    assert _noalloc(**kw) == status


def test_noalloc_limit_is_the_pair_workspace():
    """The size limit is ep_workspace_bytes of the pair against the
    scratch array's EP_NOALLOC_SCRATCH_BYTES (8 MiB): the prefill and large
    workloads fit, with room for several times their token counts."""
    lim = 8 << 20
    assert re.search(r"#define\s+EP_NOALLOC_SCRATCH_BYTES\s+\(8u << 20\)", open(HEADER).read())
    assert N.ep_workspace_bytes(4096, 8, 256, 8) <= lim
    assert N.ep_workspace_bytes(16384, 16, 384, 32) <= lim
    assert N.ep_workspace_bytes(65536, 16, 384, 32) <= lim
    assert N.ep_workspace_bytes(600000, 4, 8, 1) > lim


def _ll(**kw):
    args = dict(x=A, T=16, H=256, topk_idx=A, K=2, E=8, cap=4, quant=0, recv_x=B,
                recv_scales=None, slot=A, recv_src=A, recv_count=A, num_dropped=A,
                num_invalid=A, stream=None)
    args.update(kw)
    return N.ep_low_latency_dispatch(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(T=4097, K=1), N.EP_ERR_UNSUPPORTED),                      # T*K beyond 4096
    (dict(T=1, K=65), N.EP_ERR_UNSUPPORTED),                        # K beyond 64
    (dict(quant=3, H=8320, recv_scales=A), N.EP_ERR_UNSUPPORTED),   # per-token row of 520 pairs
    (dict(quant=2, H=4104, recv_scales=A), N.EP_ERR_UNSUPPORTED),   # 513 single pieces
    (dict(E=9000), N.EP_ERR_UNSUPPORTED),
    (dict(cap=-1), N.EP_ERR_INVALID_ARG),
    (dict(E=4096, cap=1 << 20), N.EP_ERR_INVALID_ARG),              # E*cap >= 2^31
    (dict(quant=7), N.EP_ERR_INVALID_ARG),
    (dict(quant=1, H=200, recv_scales=A), N.EP_ERR_INVALID_ARG),
    (dict(quant=1, recv_scales=None), N.EP_ERR_INVALID_ARG),
    (dict(H=12), N.EP_ERR_INVALID_ARG),
    (dict(x=A + 8), N.EP_ERR_INVALID_ARG),
    (dict(recv_count=None), N.EP_ERR_INVALID_ARG),
    (dict(num_invalid=None), N.EP_ERR_INVALID_ARG),
    (dict(num_dropped=None), N.EP_ERR_INVALID_ARG),
    (dict(slot=None), N.EP_ERR_INVALID_ARG),
    (dict(recv_x=None), N.EP_ERR_INVALID_ARG),
    (dict(K=0), N.EP_ERR_INVALID_ARG),
])
def test_low_latency_dispatch_rejects(kw, status):
    assert _ll(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(H=4), N.EP_ERR_INVALID_ARG),
    (dict(H=20), N.EP_ERR_INVALID_ARG),
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(T=-3), N.EP_ERR_INVALID_ARG),
    (dict(y=None), N.EP_ERR_INVALID_ARG),
    (dict(y_rows=-1), N.EP_ERR_INVALID_ARG),
    (dict(out=None), N.EP_ERR_INVALID_ARG),
    (dict(slot=None), N.EP_ERR_INVALID_ARG),
    (dict(out=B + 8), N.EP_ERR_INVALID_ARG),
    (dict(topk_weights=A + 1), N.EP_ERR_INVALID_ARG),
    (dict(H=(1 << 24) + 8), N.EP_ERR_UNSUPPORTED),
])
def test_combine_rejects(kw, status):
    args = dict(y=A, y_rows=32, H=256, slot=A, topk_weights=None, T=16, K=2, out=B, stream=None)
    args.update(kw)
    assert N.ep_combine(**args, check=False) == status


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), N.EP_ERR_INVALID_ARG),
    (dict(C=0), N.EP_ERR_INVALID_ARG),
    (dict(H=10), N.EP_ERR_INVALID_ARG),
    (dict(T=-1), N.EP_ERR_INVALID_ARG),
    (dict(token_indices=None), N.EP_ERR_INVALID_ARG),
    (dict(recv_x=None), N.EP_ERR_INVALID_ARG),
    (dict(tok_off=None), N.EP_ERR_INVALID_ARG),
    (dict(tok_ent=None), N.EP_ERR_INVALID_ARG),
    (dict(num_invalid=None), N.EP_ERR_INVALID_ARG),
    (dict(x=A + 4), N.EP_ERR_INVALID_ARG),
    (dict(ws=None), N.EP_ERR_WORKSPACE),
    (dict(ws_bytes=64), N.EP_ERR_WORKSPACE),
    (dict(E=1 << 16, C=1 << 16), N.EP_ERR_INVALID_ARG),
    (dict(H=(1 << 24) + 8), N.EP_ERR_UNSUPPORTED),
])
def test_ec_dispatch_rejects(kw, status):
    args = dict(x=A, T=16, H=64, token_indices=A, E=4, C=8, recv_x=B, tok_off=A, tok_ent=A,
                num_invalid=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    assert N.ep_dispatch_expert_choice(**args, check=False) == status


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), N.EP_ERR_INVALID_ARG),
    (dict(H=12), N.EP_ERR_INVALID_ARG),
    (dict(weights=None), N.EP_ERR_INVALID_ARG),
    (dict(tok_off=None), N.EP_ERR_INVALID_ARG),
    (dict(out=B + 2), N.EP_ERR_INVALID_ARG),
    (dict(H=(1 << 24) + 8), N.EP_ERR_UNSUPPORTED),
])
def test_ec_combine_rejects(kw, status):
    args = dict(y=A, weights=A, E=4, C=8, H=64, tok_off=A, tok_ent=A, T=16, out=B, stream=None)
    args.update(kw)
    assert N.ep_combine_expert_choice(**args, check=False) == status


def test_binding_raises_on_error_status():
    with pytest.raises(N.EpError):
        N.ep_combine(A, 32, 12, A, None, 16, 2, B, None)


C_USER = r"""
#include "ep.h"
#include <stdio.h>

int main(void)
{
    ep_status_t st = EP_OK;
    ep_recv_layout_t lay = EP_LAYOUT_PADDED;
    ep_quant_t q = EP_QUANT_MXFP4_E2M1;
    const int codes[] = {EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_WORKSPACE,
                         EP_ERR_HIP, EP_LAYOUT_CONTIGUOUS, EP_LAYOUT_PADDED, EP_QUANT_BF16,
                         EP_QUANT_FP8_E4M3_G128, EP_QUANT_FP8_E4M3_TOKEN, EP_QUANT_INT8_TOKEN,
                         EP_QUANT_MXFP8_E4M3, EP_QUANT_MXFP8_E5M2, EP_QUANT_MXFP4_E2M1};
    size_t b = ep_workspace_bytes(4096, 8, 256, 1) + ep_ec_workspace_bytes(8192, 64, 256);
    st = ep_get_dispatch_layout(NULL, 4, 2, 8, 1, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
    st |= ep_dispatch(NULL, 4, 64, NULL, 2, 8, NULL, lay, 8, q, NULL, NULL, NULL, NULL, NULL, NULL,
                      0, NULL);
    st |= ep_combine(NULL, 0, 64, NULL, NULL, 4, 2, NULL, NULL);
    st |= ep_dispatch_expert_choice(NULL, 4, 64, NULL, 2, 2, NULL, NULL, NULL, NULL, NULL, 0, NULL);
    st |= ep_combine_expert_choice(NULL, NULL, 2, 2, 64, NULL, NULL, 4, NULL, NULL);
    printf("%d %s %zu %d\n", (int)st, ep_status_string(EP_ERR_WORKSPACE), b,
           (int)(sizeof codes / sizeof codes[0]));
    return st == 0;    /* every call above is rejected */
}
"""


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_is_plain_c_and_links(tmp_path, std):
    """A C program that includes ep.h under strict ISO C, uses every type,
    constant and function, links against libep.so and runs: each call is an
    argument error, reported synchronously without touching a device."""
    src = tmp_path / "user.c"
    src.write_text(C_USER)
    exe = tmp_path / "user"
    lib_dir = os.path.dirname(N.LIB_PATH)
    subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe),
                    f"-L{lib_dir}", "-lep", f"-Wl,-rpath,{lib_dir}"],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    first = r.stdout.split()
    assert first[0] != "0" and "workspace" in r.stdout and first[-1] == "14"


def _pack(**kw):
    args = dict(x=A, T=16, H=256, topk_idx=A, topk_weights=A, K=2, E=8, R=4, max_rows=32,
                tokens_per_rank=A, rank_offsets=A, send_x=B, send_src=A, send_idx=A, send_w=A,
                pack_pos=A, num_dropped=A, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return N.ep_pack_by_rank(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(E=8, R=3), N.EP_ERR_INVALID_ARG),
    (dict(R=2048, E=2048), N.EP_ERR_UNSUPPORTED),
    (dict(H=12), N.EP_ERR_INVALID_ARG),
    (dict(max_rows=-1), N.EP_ERR_INVALID_ARG),
    (dict(tokens_per_rank=None), N.EP_ERR_INVALID_ARG),
    (dict(rank_offsets=None), N.EP_ERR_INVALID_ARG),
    (dict(pack_pos=None), N.EP_ERR_INVALID_ARG),
    (dict(send_x=None), N.EP_ERR_INVALID_ARG),
    (dict(send_idx=None), N.EP_ERR_INVALID_ARG),
    (dict(x=A + 8), N.EP_ERR_INVALID_ARG),
    (dict(send_w=A + 2), N.EP_ERR_INVALID_ARG),
    (dict(H=(1 << 24) + 8), N.EP_ERR_UNSUPPORTED),
    (dict(ws=None), N.EP_ERR_WORKSPACE),
    (dict(ws_bytes=64), N.EP_ERR_WORKSPACE),
])
def test_pack_rejects(kw, status):
    assert _pack(**kw) == status


def test_pack_workspace_bytes():
    assert N.ep_pack_workspace_bytes(4096, 8, 256, 8) >= 4096 * 8 * 4
    assert N.ep_pack_workspace_bytes(4096, 8, 256, 3) == 0
    assert N.ep_pack_workspace_bytes(0, 8, 256, 8) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(S=-1), N.EP_ERR_INVALID_ARG),
    (dict(K=0), N.EP_ERR_INVALID_ARG),
    (dict(H=12), N.EP_ERR_INVALID_ARG),
    (dict(partial=A + 4), N.EP_ERR_INVALID_ARG),
    (dict(partial=None), N.EP_ERR_INVALID_ARG),
    (dict(y=None), N.EP_ERR_INVALID_ARG),
])
def test_combine_partial_rejects(kw, status):
    args = dict(y=A, y_rows=64, H=256, slot=A, weights=A, S=16, K=2, partial=B, stream=None)
    args.update(kw)
    assert N.ep_combine_partial(**args, check=False) == status


@pytest.mark.parametrize("kw,status", [
    (dict(R=0), N.EP_ERR_INVALID_ARG),
    (dict(R=2048), N.EP_ERR_UNSUPPORTED),
    (dict(T=-1), N.EP_ERR_INVALID_ARG),
    (dict(H=4), N.EP_ERR_INVALID_ARG),
    (dict(pack_pos=None), N.EP_ERR_INVALID_ARG),
    (dict(out=A + 8), N.EP_ERR_INVALID_ARG),
    (dict(partial=None), N.EP_ERR_INVALID_ARG),
])
def test_combine_ranks_rejects(kw, status):
    args = dict(partial=A, rows=64, H=256, pack_pos=A, T=16, R=4, out=B, stream=None)
    args.update(kw)
    assert N.ep_combine_ranks(**args, check=False) == status
