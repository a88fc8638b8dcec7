#!/usr/bin/env python3
"""Benchmark of the MoE token dispatch/combine hot path on one MI355X.

Default workload (the headline metric): T=4096 tokens, H=7168, E=256
experts, top-8 with Zipf-skewed routing.  One step = ep_get_dispatch_layout
+ ep_dispatch (bf16, expert-contiguous receive buffer) + ep_combine (routing
weights, identity experts: y = the receive buffer).  Inputs are seeded
synthetic tensors, resident in HBM before the timed region.  W untimed
warm-up steps, then exactly K timed steps between two device
synchronisations; one JSON line is printed.

Other workloads (--workload): toy, decode (ep_low_latency_dispatch, one
launch, fp8 e4m3 with 128-channel scales into the padded [E, 128, H] buffer,
then ep_combine over bf16(q*s) rows made outside the timed region; with
--two-call the layout + dispatch pair), expert_choice (ep_dispatch_expert_choice +
ep_combine_expert_choice), large_padded.

Also reported: per-operation times (HIP events on the stream the kernels run
on, in a second pass after the timed region), a cold-cache pass (1 GiB of
scratch read before each step, outside its events, so that neither L2 nor
the 256 MB MALL holds the inputs), the roofline of the dominant
kernel (algorithmic bytes per launch over its average duration, against
8 TB/s), HBM traffic from the committed rocprofv3 counter summary when it was
taken on the current kernel sources, and the CPU oracle timed on the host on
a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
HEADLINE_METRIC = "dispatch+combine tokens/s & achieved HBM GB/s, T=4096 H=7168 E=256 top-8"


def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed, so
    that comment edits do not count as kernel changes."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] == '"':                       # string literal, kept whole
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """SHA-256 over the library sources (csrc/), comments and whitespace
    excluded: the counter summaries in profiles/ are valid while it holds."""
    d = os.path.join(ROOT, "combine_get_dispatch_04_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()


def traffic_entry(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when that summary was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("src_sha256") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- paths
class Path:
    """A workload's hot path: named operations (each a list of libep calls on
    one stream), the main kernel of each, and algorithmic bytes per op."""

    def __init__(self, name, T, ops, kernel_of, alg_bytes, meta):
        self.name, self.T, self.ops, self.kernel_of = name, T, ops, kernel_of
        self.alg_bytes, self.meta = alg_bytes, meta


# quant name -> (ep_quant_t attribute, bytes of a receive row, scale shape)
# where the scale shape maps H to (columns or 0 for one per row, numpy-like
# dtype name), or None for bf16
QUANT_MODES = {
    "bf16": ("EP_QUANT_BF16", lambda H: 2 * H, None),
    "fp8_e4m3_g128": ("EP_QUANT_FP8_E4M3_G128", lambda H: H + 4 * (H // 128),
                      lambda H: (H // 128, "float32")),
    "fp8_e4m3_token": ("EP_QUANT_FP8_E4M3_TOKEN", lambda H: H + 4, lambda H: (0, "float32")),
    "int8_token": ("EP_QUANT_INT8_TOKEN", lambda H: H + 4, lambda H: (0, "float32")),
    "mxfp8_e4m3": ("EP_QUANT_MXFP8_E4M3", lambda H: H + H // 32, lambda H: (H // 32, "uint8")),
    "mxfp8_e5m2": ("EP_QUANT_MXFP8_E5M2", lambda H: H + H // 32, lambda H: (H // 32, "uint8")),
    "mxfp4_e2m1": ("EP_QUANT_MXFP4_E2M1", lambda H: H // 2 + H // 32,
                   lambda H: (H // 32, "uint8")),
}


def dequantise(torch, recv, scales, quant, H):
    """bf16 rows from the receive buffer (identity experts), with torch
    element casts; run once, outside the timed region."""
    if quant == "bf16":
        return recv
    f8 = {"fp8_e4m3_g128": torch.float8_e4m3fn, "fp8_e4m3_token": torch.float8_e4m3fn,
          "mxfp8_e4m3": torch.float8_e4m3fn, "mxfp8_e5m2": torch.float8_e5m2}
    if quant == "int8_token":
        v = recv.view(torch.int8).float()
    elif quant == "mxfp4_e2m1":
        lut = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                            -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], device=recv.device)
        b = recv.view(torch.uint8).long()
        v = torch.stack([lut[b & 15], lut[b >> 4]], dim=-1).reshape(recv.shape[0], H)
    else:
        v = recv.view(f8[quant]).float()
    if quant == "fp8_e4m3_g128":
        v = v * scales.repeat_interleave(128, dim=1)
    elif quant in ("fp8_e4m3_token", "int8_token"):
        v = v * scales[:, None]
    else:
        v = v * torch.exp2(scales.float() - 127.0).repeat_interleave(32, dim=1)
    return v.to(torch.bfloat16)


def chunked_token_choice_path(c, N, torch, dev, sp, chunk):
    """The same step in rounds of at most `chunk` tokens (long-sequence
    chunking): each round runs layout, dispatch and combine on its slice of
    tokens, reusing one receive buffer of chunk*K rows and one workspace."""
    T, H, E, K = c.T, c.H, c.E, c.K
    if c.quant != "bf16" or c.layout != "contiguous":
        raise SystemExit("--chunk is measured for the bf16 contiguous layout")
    P = lambda t: t.data_ptr() if t is not None else None
    x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(c.topk_idx).to(dev)
    w = torch.from_numpy(c.topk_weights).to(dev)
    n_valid = int(((c.topk_idx >= 0) & (c.topk_idx < E)).sum())
    ws_bytes = N.ep_workspace_bytes(min(chunk, T), K, E, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    tpr = torch.empty(1, dtype=torch.int32, device=dev)
    itr = torch.empty((min(chunk, T), 1), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    rows = min(chunk, T) * K
    recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    slot = torch.empty((min(chunk, T), K), dtype=torch.int32, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ops = []
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        n = t1 - t0
        xs, ids, ws_, outs = x[t0:t1], idx[t0:t1], w[t0:t1], out[t0:t1]

        def layout(ids=ids, n=n):
            N.ep_get_dispatch_layout(P(ids), n, K, E, 1, P(counts), P(offsets), P(tpr), P(itr),
                                     P(ninv), P(ws), ws_bytes, sp)

        def dispatch(xs=xs, ids=ids, n=n):
            N.ep_dispatch(P(xs), n, H, P(ids), K, E, P(offsets), N.EP_LAYOUT_CONTIGUOUS, n * K,
                          N.EP_QUANT_BF16, P(recv), None, P(slot), P(src), P(nd), P(ws),
                          ws_bytes, sp)

        def combine(ws_=ws_, outs=outs, n=n):
            N.ep_combine(P(recv), n * K, H, P(slot), P(ws_), n, K, P(outs), sp)

        ops += [("layout", layout), ("dispatch", dispatch), ("combine", combine)]
    alg = {"layout": T * K * 4,
           "dispatch": T * H * 2 + n_valid * 2 * H + 2 * T * K * 4,
           "combine": n_valid * H * 2 + T * H * 2 + 2 * T * K * 4}
    kern = {"layout": "layout_chunk_kernel", "dispatch": "dispatch_kernel",
            "combine": "combine_kernel"}
    meta = {"T": T, "H": H, "E": E, "top_k": K, "recv_layout": "contiguous", "quant": "bf16",
            "combine": "weighted", "valid_slots": n_valid, "chunk_tokens": chunk,
            "rounds": (T + chunk - 1) // chunk, "receive_rows": rows}
    return Path(c.name, T, ops, kern, alg, meta)


def token_choice_path(c, N, torch, dev, sp):
    T, H, E, K = c.T, c.H, c.E, c.K
    quant = c.quant
    qname, row_bytes, scale_shape = QUANT_MODES[quant]
    padded = c.layout == "padded"
    cap_or_rows = c.cap if padded else T * K
    rows = E * c.cap if padded else T * K
    P = lambda t: t.data_ptr() if t is not None else None
    x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(c.topk_idx).to(dev)
    w = torch.from_numpy(c.topk_weights).to(dev)
    n_valid = int(((c.topk_idx >= 0) & (c.topk_idx < E)).sum())
    ws_bytes = N.ep_workspace_bytes(T, K, E, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    tpr = torch.empty(1, dtype=torch.int32, device=dev)
    itr = torch.empty((T, 1), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    if quant == "bf16":
        recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
        scales = None
    else:
        recv = torch.empty((rows, H // 2 if quant == "mxfp4_e2m1" else H), dtype=torch.uint8,
                           device=dev)
        ncol, sdt = scale_shape(H)
        scales = torch.empty((rows, ncol) if ncol else (rows,), dtype=getattr(torch, sdt),
                             device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    qcode = getattr(N, qname)
    lay = N.EP_LAYOUT_PADDED if padded else N.EP_LAYOUT_CONTIGUOUS

    def layout():
        N.ep_get_dispatch_layout(P(idx), T, K, E, 1, P(counts), P(offsets), P(tpr), P(itr),
                                 P(ninv), P(ws), ws_bytes, sp)

    def dispatch():
        N.ep_dispatch(P(x), T, H, P(idx), K, E, P(offsets), lay, cap_or_rows, qcode, P(recv),
                      P(scales), P(slot), P(src), P(nd), P(ws), ws_bytes, sp)

    if quant != "bf16":
        # identity expert on the dequantised rows, built once outside the timed region
        layout()
        dispatch()
        torch.cuda.synchronize()
        y = dequantise(torch, recv, scales, quant, H)
        torch.cuda.synchronize()
    else:
        y = recv

    def combine():
        N.ep_combine(P(y), rows, H, P(slot), P(w), T, K, P(out), sp)

    alg = {"layout": T * K * 4,
           "dispatch": T * H * 2 + n_valid * row_bytes(H) + 2 * T * K * 4,
           "combine": n_valid * H * 2 + T * H * 2 + 2 * T * K * 4}
    kern = {"layout": "layout_chunk_kernel",
            "dispatch": "dispatch_kernel", "combine": "combine_kernel"}
    meta = {"T": T, "H": H, "E": E, "top_k": K, "recv_layout": c.layout, "quant": quant,
            "cap": c.cap, "combine": "weighted", "valid_slots": n_valid}
    return Path(c.name, T, [("layout", layout), ("dispatch", dispatch), ("combine", combine)],
                kern, alg, meta)


def low_latency_path(c, N, torch, dev, sp):
    """The decode step as its caller makes it: ep_low_latency_dispatch (one
    launch: ranks, codes, scales and counts) into the padded [E, cap] rows,
    then ep_combine."""
    T, H, E, K, cap = c.T, c.H, c.E, c.K, c.cap
    quant = c.quant
    qname, row_bytes, scale_shape = QUANT_MODES[quant]
    rows = E * cap
    P = lambda t: t.data_ptr() if t is not None else None
    x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(c.topk_idx).to(dev)
    w = torch.from_numpy(c.topk_weights).to(dev)
    n_valid = int(((c.topk_idx >= 0) & (c.topk_idx < E)).sum())
    if quant == "bf16":
        recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
        scales = None
    else:
        recv = torch.empty((rows, H // 2 if quant == "mxfp4_e2m1" else H), dtype=torch.uint8,
                           device=dev)
        ncol, sdt = scale_shape(H)
        scales = torch.empty((rows, ncol) if ncol else (rows,), dtype=getattr(torch, sdt),
                             device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    qcode = getattr(N, qname)

    def dispatch():
        N.ep_low_latency_dispatch(P(x), T, H, P(idx), K, E, cap, qcode, P(recv), P(scales),
                                  P(slot), P(src), P(cnt), P(nd), P(ninv), sp)

    if quant != "bf16":
        # identity expert on the dequantised rows, built once outside the timed region
        dispatch()
        torch.cuda.synchronize()
        y = dequantise(torch, recv, scales, quant, H)
        torch.cuda.synchronize()
    else:
        y = recv

    def combine():
        N.ep_combine(P(y), rows, H, P(slot), P(w), T, K, P(out), sp)

    alg = {"dispatch": T * H * 2 + n_valid * row_bytes(H) + 2 * T * K * 4 + E * 4,
           "combine": n_valid * H * 2 + T * H * 2 + 2 * T * K * 4}
    kern = {"dispatch": "dispatch_kernel", "combine": "combine_kernel"}
    meta = {"T": T, "H": H, "E": E, "top_k": K, "recv_layout": "padded", "quant": quant,
            "cap": cap, "combine": "weighted", "valid_slots": n_valid,
            "dispatch": "ep_low_latency_dispatch (one launch)"}
    return Path(c.name, T, [("dispatch", dispatch), ("combine", combine)], kern, alg, meta)


def expert_choice_path(c, N, torch, dev, sp):
    T, H, E, C = c.T, c.H, c.E, c.C
    P = lambda t: t.data_ptr()
    x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
    ti = torch.from_numpy(c.token_indices).to(dev)
    w = torch.from_numpy(c.weights).to(dev)
    ws_bytes = N.ep_ec_workspace_bytes(T, E, C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    recv = torch.empty((E, C, H), dtype=torch.bfloat16, device=dev)
    off = torch.empty(T + 1, dtype=torch.int32, device=dev)
    ent = torch.empty(E * C, dtype=torch.int32, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    flat = c.token_indices.ravel()
    valid = flat[(flat >= 0) & (flat < T)]
    n_valid, U = int(valid.size), int(np.unique(valid).size)

    def dispatch():
        N.ep_dispatch_expert_choice(P(x), T, H, P(ti), E, C, P(recv), P(off), P(ent), P(ninv),
                                    P(ws), ws_bytes, sp)

    def combine():
        N.ep_combine_expert_choice(P(recv), P(w), E, C, H, P(off), P(ent), T, P(out), sp)

    alg = {"dispatch": U * H * 2 + n_valid * H * 2 + E * C * 4 + (T + 1) * 4 + n_valid * 4,
           "combine": n_valid * H * 2 + T * H * 2 + E * C * 4 + (T + 1) * 4 + n_valid * 4}
    kern = {"dispatch": "ec_dispatch_fused_kernel", "combine": "ec_combine_kernel"}
    meta = {"T": T, "H": H, "E": E, "capacity": C, "valid_entries": n_valid,
            "distinct_tokens": U}
    return Path(c.name, T, [("dispatch", dispatch), ("combine", combine)], kern, alg, meta)


def cpu_baseline(c, budget_s):
    """The oracle as it stands (single thread) on full passes of the same
    workload until `budget_s` seconds have elapsed."""
    import oracle
    reps = 0
    t0 = time.perf_counter()
    while True:
        if hasattr(c, "token_indices"):
            recv, _ = oracle.ec_dispatch(c.x, c.token_indices)
            oracle.ec_invert(c.token_indices, c.T)
            oracle.ec_combine(recv, c.weights, c.token_indices, c.T)
            what = "expert-choice dispatch, inverse map, weighted combine"
        else:
            padded = c.layout == "padded"
            cap = c.cap if padded else c.T * c.K
            rows = c.E * c.cap if padded else c.T * c.K
            oracle.layout(c.topk_idx, c.E)
            slot, _, _ = oracle.slots(c.topk_idx, c.E, padded, cap)
            if c.quant == "bf16":
                y = oracle.dispatch_bf16(c.x, slot, rows)
            else:
                if c.quant == "fp8_e4m3_g128":
                    oracle.dispatch_fp8(c.x, slot, rows)
                elif c.quant in oracle.TOKEN_FMT:
                    oracle.dispatch_token_quant(c.x, slot, rows, c.quant)
                else:
                    oracle.dispatch_mx(c.x, slot, rows, c.quant)
                y = np.zeros((rows, c.H), np.uint16)
            oracle.combine(y, slot, c.topk_weights)
            what = "layout, slots, dispatch, weighted combine"
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": reps * c.T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full pass(es) of the same workload ({what}; {c.T} tokens each), "
                      f"{el:.1f} s on one host thread",
            "host_cpu": host_cpu_model(), "host_logical_cpus": os.cpu_count()}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def inputs_sha256(c):
    """SHA-256 of every input array, as handed to both the GPU path and the oracle."""
    names = ("x", "token_indices", "weights") if hasattr(c, "token_indices") else \
            ("x", "topk_idx", "topk_weights")
    return {n: hashlib.sha256(np.ascontiguousarray(getattr(c, n)).tobytes()).hexdigest()
            for n in names}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "toy", "decode", "expert_choice", "large_padded", "expert_choice_tc"])
    ap.add_argument("--quant", default=None, choices=sorted(QUANT_MODES),
                    help="dispatch quantisation of a token-choice workload (default: the "
                         "workload's own: bf16, or fp8_e4m3_g128 for decode)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="run a token-choice step in rounds of at most this many tokens "
                         "(0 = one round)")
    ap.add_argument("--two-call", action="store_true",
                    help="decode: ep_get_dispatch_layout + ep_dispatch (padded) instead of "
                         "the one-launch ep_low_latency_dispatch")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="cold pass: read this many MiB of scratch before each step, "
                         "outside the step's events (0 = no cold pass)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): the multi-GPU "
              "exchange is not built", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_get_dispatch_04_amd._native as N
    from combine_get_dispatch_04_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    c = W.WORKLOADS[a.workload]()
    if a.quant is not None:
        if a.workload == "expert_choice":
            print("--quant applies to token-choice workloads only", file=sys.stderr)
            sys.exit(2)
        c.quant = a.quant
    if a.workload == "expert_choice":
        path = expert_choice_path(c, N, torch, dev, sp)
    elif a.chunk > 0:
        path = chunked_token_choice_path(c, N, torch, dev, sp, a.chunk)
    elif a.workload == "decode" and not a.two_call:
        path = low_latency_path(c, N, torch, dev, sp)
    else:
        path = token_choice_path(c, N, torch, dev, sp)
    if a.copy_probe_mib:
        src = torch.ones(a.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1, out=dst)          # an elementwise kernel: reads and writes N MiB
        torch.cuda.synchronize()
        del src, dst

    def step():
        for _, fn in path.ops:
            fn()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps between two device synchronisations, with
    # no per-operation events inside (an event record costs the stream a few
    # microseconds, about 13 us per step for four of them)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(a.steps):
        step()
    r1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / a.steps
    region_ms = r0.elapsed_time(r1) / a.steps

    # per-operation durations: a second pass of K steps with HIP events
    # around each operation on the stream the kernels run on
    nops = len(path.ops)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nops + 1)] for _ in range(a.steps)]
    for i in range(a.steps):
        e = ev[i]
        for j, (_, fn) in enumerate(path.ops):
            e[j].record(stream)
            fn()
        e[nops].record(stream)
    torch.cuda.synchronize()
    op_us, launches = {}, {}
    for j, (name, _) in enumerate(path.ops):       # a chunked step repeats each name
        op_us[name] = op_us.get(name, 0.0) + float(
            np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]) * 1e3)
        launches[name] = launches.get(name, 0) + 1
    step_ev = np.array([e[0].elapsed_time(e[nops]) for e in ev]) * 1e3

    # cold pass: before each step (outside its events) read flush_mib MiB of
    # scratch, which evicts L2 and the 256 MB MALL; a read leaves clean lines
    # behind, so the step does not pay for writing back the flush.  The
    # scratch is allocated and filled only now: written at start-up, it
    # slowed the timed pass of the chunked workload by 41 us per step
    # (204.5 -> 245.8 us) although that pass never touches it.
    cold = None
    if a.flush_mib:
        flush = torch.ones(a.flush_mib << 20, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(a.steps)]
        for i in range(a.steps):
            flush.sum(dtype=torch.int64)
            cev[i][0].record(stream)
            step()
            cev[i][1].record(stream)
        torch.cuda.synchronize()
        cus = np.array([b_.elapsed_time(e_) for b_, e_ in cev]) * 1e3
        med = float(np.median(cus))
        cold = {"flush_mib": a.flush_mib, "us_per_step_median": med,
                "us_per_step_p10": float(np.percentile(cus, 10)),
                "us_per_step_p90": float(np.percentile(cus, 90)),
                "tokens_per_s": path.T / (med * 1e-6),
                "achieved_GBps": sum(path.alg_bytes.values()) / (med * 1e-6) / 1e9}

    alg_total = sum(path.alg_bytes.values())
    dom = max(("dispatch", "combine"), key=lambda n: op_us[n])
    dom_us, dom_bytes = op_us[dom] / launches[dom], path.alg_bytes[dom] / launches[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    headline = (a.workload == "prefill" and path.meta.get("quant") == "bf16"
                and "chunk_tokens" not in path.meta)
    res = {
        "metric": HEADLINE_METRIC if headline else
                  f"dispatch+combine tokens/s & achieved HBM GB/s, {c.name}"
                  + (f" ({path.meta['quant']})" if path.meta.get("quant", "bf16") != "bf16" else "")
                  + (f" (rounds of {path.meta['chunk_tokens']} tokens)"
                     if "chunk_tokens" in path.meta else ""),
        "value": path.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if path.meta.get("quant", "bf16") == "bf16" else
                 f"{path.meta['quant']} dispatch, bf16 combine",
        "data": "synthetic",
        "config": {"workload": c.name, **path.meta},
        "achieved_GBps": alg_total / (ms_per_step * 1e-3) / 1e9,
        "frac_of_peak_hbm": alg_total / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "algorithmic_bytes_per_step": alg_total,
        "algorithmic_bytes_per_op": path.alg_bytes,
        "timed_region_event_ms_per_step": region_ms,
        "per_op_us": {**op_us, "step_with_op_events": float(step_ev.mean()),
                      "step_with_op_events_p10": float(np.percentile(step_ev, 10)),
                      "step_with_op_events_p90": float(np.percentile(step_ev, 90))},
        "roofline": {"bound": "hbm", "kernel": path.kernel_of[dom], "op": dom,
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic_entry(a.workload, path.kernel_of[dom]),
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": dom_us},
    }
    res["cold"] = cold
    res["inputs_sha256"] = inputs_sha256(c)
    if a.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(c, a.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
