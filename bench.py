#!/usr/bin/env python3
"""Benchmark of the MoE token dispatch/combine hot path on one MI355X.

Default workload (the headline metric): T=4096 tokens, H=7168, E=256
experts, top-8 with Zipf-skewed routing.  One step = ep_get_dispatch_layout
+ ep_dispatch (bf16, expert-contiguous receive buffer) + ep_combine (routing
weights, identity experts: y = the receive buffer).  Inputs are seeded
synthetic tensors, resident in HBM before the timed region.  W untimed
warm-up steps, then exactly K timed steps between two device
synchronisations; one JSON line is printed.

Other workloads (--workload): toy, decode (fp8 e4m3 with 128-channel scales
into the padded [E, 128, H] buffer; combine reads bf16(q*s) rows made
outside the timed region), expert_choice (ep_dispatch_expert_choice +
ep_combine_expert_choice), large_padded.

Also reported: per-operation times (HIP events on the stream the kernels run
on, in a second pass after the timed region), a cold-cache pass (1 GiB of
scratch written before each step, outside its events, so that neither L2 nor
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


def kernel_source_hash():
    d = os.path.join(ROOT, "combine_get_dispatch_04_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
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


def token_choice_path(c, N, torch, dev, sp):
    T, H, E, K = c.T, c.H, c.E, c.K
    fp8 = c.quant == "fp8_e4m3_g128"
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
    recv = torch.empty((rows, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    scales = torch.empty((rows, H // 128), dtype=torch.float32, device=dev) if fp8 else None
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    quant = N.EP_QUANT_FP8_E4M3_G128 if fp8 else N.EP_QUANT_BF16
    lay = N.EP_LAYOUT_PADDED if padded else N.EP_LAYOUT_CONTIGUOUS

    def layout():
        N.ep_get_dispatch_layout(P(idx), T, K, E, 1, P(counts), P(offsets), P(tpr), P(itr),
                                 P(ninv), P(ws), ws_bytes, sp)

    def dispatch():
        N.ep_dispatch(P(x), T, H, P(idx), K, E, P(offsets), lay, cap_or_rows, quant, P(recv),
                      P(scales), P(slot), P(src), P(nd), P(ws), ws_bytes, sp)

    if fp8:
        # identity expert on the dequantised rows, built once outside the timed region
        layout()
        dispatch()
        torch.cuda.synchronize()
        y = (recv.view(torch.float8_e4m3fn).float()
             * scales.repeat_interleave(128, dim=1)).to(torch.bfloat16)
        torch.cuda.synchronize()
    else:
        y = recv

    def combine():
        N.ep_combine(P(y), rows, H, P(slot), P(w), T, K, P(out), sp)

    row_in = H + 4 * (H // 128) if fp8 else H * 2
    alg = {"layout": T * K * 4,
           "dispatch": T * H * 2 + n_valid * row_in + 2 * T * K * 4,
           "combine": n_valid * H * 2 + T * H * 2 + 2 * T * K * 4}
    kern = {"layout": "layout_chunk_kernel",
            "dispatch": "dispatch_kernel", "combine": "combine_kernel"}
    meta = {"T": T, "H": H, "E": E, "top_k": K, "recv_layout": c.layout, "quant": c.quant,
            "cap": c.cap, "combine": "weighted", "valid_slots": n_valid}
    return Path(c.name, T, [("layout", layout), ("dispatch", dispatch), ("combine", combine)],
                kern, alg, meta)


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
            if c.quant == "fp8_e4m3_g128":
                oracle.dispatch_fp8(c.x, slot, rows)
                y = np.zeros((rows, c.H), np.uint16)
            else:
                y = oracle.dispatch_bf16(c.x, slot, rows)
            oracle.combine(y, slot, c.topk_weights)
            what = "layout, slots, dispatch, weighted combine"
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": reps * c.T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full pass(es) of the same workload ({what}; {c.T} tokens each), "
                      f"{el:.1f} s on one host thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "toy", "decode", "expert_choice", "large_padded"])
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="cold pass: write this many MiB of scratch before each step, "
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
    if a.workload == "expert_choice":
        path = expert_choice_path(c, N, torch, dev, sp)
    else:
        path = token_choice_path(c, N, torch, dev, sp)
    flush = torch.empty(a.flush_mib << 20, dtype=torch.uint8, device=dev) if a.flush_mib else None
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
    op_us = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]) * 1e3)
             for j, (name, _) in enumerate(path.ops)}
    step_ev = np.array([e[0].elapsed_time(e[nops]) for e in ev]) * 1e3

    # cold pass: before each step (outside its events) write flush_mib MiB of
    # scratch, which evicts L2 and the 256 MB MALL
    cold = None
    if flush is not None:
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(a.steps)]
        for i in range(a.steps):
            flush.fill_(i & 0xFF)
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
    dom_us, dom_bytes = op_us[dom], path.alg_bytes[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    headline = a.workload == "prefill"
    res = {
        "metric": HEADLINE_METRIC if headline else
                  f"dispatch+combine tokens/s & achieved HBM GB/s, {c.name}",
        "value": path.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 dispatch, bf16 combine" if a.workload == "decode" else "bf16",
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
    if a.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(c, a.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
