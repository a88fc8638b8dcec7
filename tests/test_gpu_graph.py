"""The hot path captured in a HIP graph and replayed.

Layout, dispatch and combine (and the expert-choice and low-latency pairs,
and one rank's share of the exchange) are recorded once through the torch
front end (the C ABI enqueues everything on the current stream, allocates
nothing and issues no memset), then the graph is replayed with new inputs
copied into its static tensors.  Between replays the same
calls run eagerly on the new inputs, with synchronisations, and every replay
must give the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

from combine_get_dispatch_04_amd import api
from combine_get_dispatch_04_amd import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _dev_tc(c):
    x = torch.from_numpy(c.x.view(np.int16)).cuda().view(torch.bfloat16)
    return x, torch.from_numpy(c.topk_idx).cuda(), torch.from_numpy(c.topk_weights).cuda()


def _tc_step(x, idx, w, E, quant):
    L = api.get_dispatch_layout(idx, E)
    recv, scales, h = api.dispatch(x, L, quant=quant)
    out = api.combine(recv, h, w) if quant == "bf16" else None
    return dict(counts=L.num_tokens_per_expert, offsets=L.offsets, slot=h.slot,
                recv_src=h.recv_src, recv=recv, scales=scales, out=out)


def _same(g, e):
    """Everything the call defines: layout, slots, and the rows, sources and
    scales of the slots that were written (other receive rows are left as
    they were), and the combine output."""
    b = lambda t: t.view(torch.uint8)
    if not (torch.equal(g["counts"], e["counts"]) and torch.equal(g["offsets"], e["offsets"])
            and torch.equal(g["slot"], e["slot"])):
        return False
    kept = e["slot"][e["slot"] >= 0].long()
    if not (torch.equal(g["recv_src"][kept], e["recv_src"][kept])
            and torch.equal(b(g["recv"][kept]), b(e["recv"][kept]))):
        return False
    if e["scales"] is not None and not torch.equal(b(g["scales"][kept]), b(e["scales"][kept])):
        return False
    return e["out"] is None or torch.equal(b(g["out"]), b(e["out"]))


# (T, H, E, K, quant): one layout chunk; and 64 chunks over E = 384, whose
# column scan takes more than 64 KiB of LDS (the launch path that sets the
# kernel's shared-memory attribute)
TC_GRAPH = [(777, 1024, 64, 6, "bf16"), (777, 1024, 64, 6, "fp8_e4m3_g128"),
            (4096, 64, 384, 16, "bf16")]


@pytest.mark.parametrize("T,H,E,K,quant", TC_GRAPH)
def test_token_choice_graph_replays(T, H, E, K, quant):
    x_s, idx_s, w_s = _dev_tc(W.random_token_choice(50, T, H, E, K, p_pad=0.1, p_invalid=0.02))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up off the capture
        _tc_step(x_s, idx_s, w_s, E, quant)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_out = _tc_step(x_s, idx_s, w_s, E, quant)
    for r in range(REPLAYS):
        x, idx, w = _dev_tc(W.random_token_choice(60 + r, T, H, E, K, p_pad=0.1,
                                                  p_invalid=0.02, p_dup=0.1))
        x_s.copy_(x)
        idx_s.copy_(idx)
        w_s.copy_(w)
        g.replay()
        torch.cuda.synchronize()
        eager = _tc_step(x, idx, w, E, quant)
        torch.cuda.synchronize()
        assert _same(graph_out, eager), r


# (T, H, E, C): the inverse map inside the copy's launch; and in a launch
# of its own with 104000 B of LDS
EC_GRAPH = [(1500, 512, 16, 64), (13000, 8, 8, 1000)]


@pytest.mark.parametrize("T,H,E,C", EC_GRAPH)
def test_expert_choice_graph_replays(T, H, E, C):
    def inputs(seed):
        c = W.random_expert_choice(seed, T, H, E, C, p_empty=0.1, hot=5)
        return (torch.from_numpy(c.x.view(np.int16)).cuda().view(torch.bfloat16),
                torch.from_numpy(c.token_indices).cuda(), torch.from_numpy(c.weights).cuda())

    def step(x, ti, w):
        recv, h = api.dispatch_expert_choice(x, ti, w)
        return [h.tok_off, h.tok_ent, recv, api.combine_expert_choice(recv, h)]

    x_s, ti_s, w_s = inputs(70)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(x_s, ti_s, w_s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_out = step(x_s, ti_s, w_s)
    for r in range(REPLAYS):
        x, ti, w = inputs(80 + r)
        x_s.copy_(x)
        ti_s.copy_(ti)
        w_s.copy_(w)
        g.replay()
        torch.cuda.synchronize()
        eager = step(x, ti, w)
        torch.cuda.synchronize()
        n = int(eager[0][-1].item())            # entries beyond tok_off[T] are not written
        assert torch.equal(graph_out[0], eager[0]), r
        assert torch.equal(graph_out[1][:n], eager[1][:n]), r
        filled = ((ti >= 0) & (ti < T)).reshape(-1)
        assert torch.equal(graph_out[2].reshape(E * C, H)[filled].view(torch.int16),
                           eager[2].reshape(E * C, H)[filled].view(torch.int16)), r
        assert torch.equal(graph_out[3].view(torch.int16), eager[3].view(torch.int16)), r


# (T, H, E, K, cap, quant): the decode shape with overflow, fp8 and bf16
LL_GRAPH = [(128, 7168, 256, 8, 6, "fp8_e4m3_g128"), (96, 1024, 32, 6, 16, "bf16")]


@pytest.mark.parametrize("T,H,E,K,cap,quant", LL_GRAPH)
def test_low_latency_graph_replays(T, H, E, K, cap, quant):
    """low_latency_dispatch (one launch) + low_latency_combine captured."""
    def step(x, idx, w):
        recv, scales, h = api.low_latency_dispatch(x, idx, cap, E, quant=quant)
        out = api.low_latency_combine(recv, idx, w, h) if quant == "bf16" else None
        return dict(slot=h.slot, recv_src=h.recv_src, cnt=h.recv_count, nd=h.num_dropped,
                    ninv=h.num_invalid, recv=recv.reshape(E * cap, -1),
                    scales=None if scales is None else scales.reshape(E * cap, -1), out=out)

    x_s, idx_s, w_s = _dev_tc(W.random_token_choice(90, T, H, E, K, p_pad=0.1, p_invalid=0.02))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(x_s, idx_s, w_s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        go = step(x_s, idx_s, w_s)
    b = lambda t: t.view(torch.uint8)
    for r in range(REPLAYS):
        x, idx, w = _dev_tc(W.random_token_choice(100 + r, T, H, E, K, p_pad=0.1,
                                                  p_invalid=0.02, p_dup=0.1))
        x_s.copy_(x)
        idx_s.copy_(idx)
        w_s.copy_(w)
        g.replay()
        torch.cuda.synchronize()
        e = step(x, idx, w)
        torch.cuda.synchronize()
        for k in ("slot", "cnt", "nd", "ninv"):
            assert torch.equal(go[k], e[k]), (r, k)
        kept = e["slot"][e["slot"] >= 0].long()
        assert torch.equal(go["recv_src"][kept], e["recv_src"][kept]), r
        assert torch.equal(b(go["recv"][kept]), b(e["recv"][kept])), r
        if e["scales"] is not None:
            assert torch.equal(b(go["scales"][kept]), b(e["scales"][kept])), r
        if e["out"] is not None:
            assert torch.equal(b(go["out"]), b(e["out"])), r


# (T, H, E, K, R): one rank's share of the exchange at R = 8 and R = 4
RANK_GRAPH = [(600, 512, 64, 6, 8), (300, 1024, 32, 8, 4)]


@pytest.mark.parametrize("T,H,E,K,R", RANK_GRAPH)
def test_rank_share_graph_replays(T, H, E, K, R):
    """pack_by_rank, the receiver's layout + scatter of every packed row,
    combine_partial and combine_ranks captured as one step.  The routing is
    fixed (so the packed row count S, sized on the host, is too); x and the
    weights change on every replay."""
    c = W.random_token_choice(130, T, H, E, K, p_pad=0.1, p_invalid=0.02)
    per = E // R
    ids = c.topk_idx
    ok = (ids >= 0) & (ids < E)
    S = int(sum(len(set((row[m] // per).tolist())) for row, m in zip(ids, ok)))

    def step(x, idx, w):
        pk = api.pack_by_rank(x, idx, E, R, topk_weights=w, max_rows=S)
        _, recv, _, h = api.receive(pk.send_x, pk.send_idx, per)
        part = api.combine_partial(recv, h, pk.send_w)
        out = api.combine_ranks(part, pk)
        return dict(tpr=pk.num_tokens_per_rank, off=pk.rank_offsets, sx=pk.send_x,
                    src=pk.send_src, sidx=pk.send_idx, sw=pk.send_w, pos=pk.pack_pos,
                    nd=pk.num_dropped, slot=h.slot, recv=recv, part=part, out=out)

    x_s, idx_s, w_s = _dev_tc(c)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(x_s, idx_s, w_s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        go = step(x_s, idx_s, w_s)
    b = lambda t: t.view(torch.uint8)
    for r in range(REPLAYS):
        c2 = W.random_token_choice(140 + r, T, H, E, K)
        x = torch.from_numpy(c2.x.view(np.int16)).cuda().view(torch.bfloat16)
        w = torch.from_numpy(c2.topk_weights).cuda()
        x_s.copy_(x)
        w_s.copy_(w)
        g.replay()
        torch.cuda.synchronize()
        e = step(x, idx_s, w)
        torch.cuda.synchronize()
        assert int(e["nd"][0]) == 0, r
        for k in ("tpr", "off", "src", "sidx", "pos", "nd", "slot"):
            assert torch.equal(go[k], e[k]), (r, k)
        for k in ("sx", "sw", "part", "out"):
            assert torch.equal(b(go[k]), b(e[k])), (r, k)
        kept = e["slot"][e["slot"] >= 0].long()           # receive rows that were written
        assert torch.equal(b(go["recv"][kept]), b(e["recv"][kept])), r
