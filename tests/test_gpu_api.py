"""The torch front end (combine_get_dispatch_04_amd.api) against the oracle,
and its argument checks.

Each Buffer-style call of "DeepEP-Ascend" README, API Overview
(get_dispatch_layout, dispatch in the contiguous and the low-latency padded
form, combine) and the expert-centric pair of "[Feature Request] Support
Expert-Choice Routing via Native Expert-Centric API", Solution 1, is run on
seeded inputs and compared with the oracle: integers and codes bit for bit,
combines within |gpu - oracle| <= 2^-7 |oracle| + 1e-3.  The checks of bad
arguments raise before anything is launched.
"""
import numpy as np
import pytest
import torch

import brute
import gpu_util as G
import oracle
from combine_get_dispatch_04_amd import api
from combine_get_dispatch_04_amd import workloads as W

pytestmark = pytest.mark.gpu


def _tc(seed, T=300, H=512, E=24, K=4):
    c = W.random_token_choice(seed, T, H, E, K, p_pad=0.1, p_invalid=0.02, p_dup=0.1)
    return c, G.dev(c.x), G.dev(c.topk_idx), G.dev(c.topk_weights)


def _written(slot, rows):
    m = np.zeros(rows, bool)
    m[slot[slot >= 0]] = True
    return m


def test_layout_matches_oracle():
    c, _, idx, _ = _tc(1, E=32)
    L = api.get_dispatch_layout(idx, c.E, num_ranks=4)
    torch.cuda.synchronize()
    ref = oracle.layout(c.topk_idx, c.E, 4)
    assert np.array_equal(G.host(L.num_tokens_per_expert), ref["counts"])
    assert np.array_equal(G.host(L.offsets), ref["offsets"])
    assert np.array_equal(G.host(L.num_tokens_per_rank), ref["tokens_per_rank"])
    assert np.array_equal(G.host(L.is_token_in_rank), ref["is_token_in_rank"])
    assert int(G.host(L.num_invalid)[0]) == ref["num_invalid"]
    assert L.num_tokens_per_rdma_rank is None


@pytest.mark.parametrize("recv_layout", ["contiguous", "padded"])
def test_bf16_round_trip(recv_layout):
    c, x, idx, w = _tc(2)
    L = api.get_dispatch_layout(idx, c.E)
    cap = 30 if recv_layout == "padded" else None
    recv, scales, h = api.dispatch(x, L, recv_layout=recv_layout, cap=cap)
    out = api.combine(recv, h, w)
    torch.cuda.synchronize()
    padded = recv_layout == "padded"
    s_ref, src_ref, nd_ref = oracle.slots(c.topk_idx, c.E, padded, cap if padded else c.T * c.K)
    assert scales is None and h.rows == recv.shape[0]
    assert np.array_equal(G.host(h.slot), s_ref)
    assert int(G.host(h.num_dropped)[0]) == nd_ref
    rows = h.rows
    m = _written(s_ref, rows)
    y = oracle.dispatch_bf16(c.x, s_ref, rows)
    assert np.array_equal(G.host(recv)[m], y[m])
    assert np.array_equal(G.host(h.recv_src)[m], src_ref[m])
    G.assert_combine_close(G.host(out), oracle.combine(y, s_ref, c.topk_weights))


@pytest.mark.parametrize("quant,mode", [("fp8_e4m3_g128", None), ("int8", "int8_token"),
                                        ("pertoken_fp8_e4m3", "fp8_e4m3_token"),
                                        ("mx_fp8_e5m2", "mxfp8_e5m2"),
                                        ("mx_fp4_e2m1", "mxfp4_e2m1")])
def test_quantised_dispatch_and_aliases(quant, mode):
    c, x, idx, _ = _tc(3)
    L = api.get_dispatch_layout(idx, c.E)
    recv, scales, h = api.dispatch(x, L, quant=quant)
    torch.cuda.synchronize()
    s_ref, _, _ = oracle.slots(c.topk_idx, c.E, False, c.T * c.K)
    rows = c.T * c.K
    if mode is None:
        q, s = oracle.dispatch_fp8(c.x, s_ref, rows)
    elif mode in oracle.TOKEN_FMT:
        q, s = oracle.dispatch_token_quant(c.x, s_ref, rows, mode)
    else:
        q, s = oracle.dispatch_mx(c.x, s_ref, rows, mode)
    m = _written(s_ref, rows)
    got_q = recv.view(torch.uint8).cpu().numpy()
    want = np.ascontiguousarray(q[m]).view(np.uint8).reshape(got_q[m].shape)
    assert np.array_equal(got_q[m], want)
    got_s = scales.cpu().numpy()
    if got_s.dtype == np.float32:
        assert np.array_equal(got_s[m].view(np.uint32), s[m].view(np.uint32))
    else:
        assert np.array_equal(got_s[m], s[m])


def test_combine_into_given_out_and_unit_weights():
    c, x, idx, _ = _tc(4)
    L = api.get_dispatch_layout(idx, c.E)
    recv, _, h = api.dispatch(x, L)
    out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device="cuda")
    r = api.combine(recv, h, None, out=out)
    torch.cuda.synchronize()
    assert r.data_ptr() == out.data_ptr()
    s_ref, _, _ = oracle.slots(c.topk_idx, c.E, False, c.T * c.K)
    y = oracle.dispatch_bf16(c.x, s_ref, c.T * c.K)
    G.assert_combine_close(G.host(out), oracle.combine(y, s_ref, None))


def test_expert_choice_round_trip():
    c = W.random_expert_choice(5, 700, 256, 12, 40, p_empty=0.1, hot=6)
    x, ti, w = G.dev(c.x), G.dev(c.token_indices), G.dev(c.weights)
    recv, h = api.dispatch_expert_choice(x, ti, w)
    out = api.combine_expert_choice(recv, h)
    torch.cuda.synchronize()
    r_ref, ninv = oracle.ec_dispatch(c.x, c.token_indices)
    off, ent = oracle.ec_invert(c.token_indices, c.T)
    assert int(G.host(h.num_invalid)[0]) == ninv
    assert np.array_equal(G.host(h.tok_off), off)
    n = int(off[-1])
    assert np.array_equal(G.host(h.tok_ent)[:n], ent[:n])
    filled = ((c.token_indices >= 0) & (c.token_indices < c.T)).reshape(-1)
    got = G.host(recv).reshape(-1, c.H)
    assert np.array_equal(got[filled], r_ref.reshape(-1, c.H)[filled])
    G.assert_combine_close(G.host(out), oracle.ec_combine(r_ref, c.weights, c.token_indices, c.T))


def test_bad_arguments_raise_before_launch():
    c, x, idx, w = _tc(6, T=64, H=256, E=8, K=2)
    L = api.get_dispatch_layout(idx, c.E)
    recv, _, h = api.dispatch(x, L)
    torch.cuda.synchronize()
    bf = dict(dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out must be"):
        api.combine(recv, h, w, out=torch.empty((c.T - 1, c.H), **bf))
    with pytest.raises(ValueError, match="out must be"):
        api.combine(recv, h, w, out=torch.empty((c.T, 2 * c.H), **bf))
    with pytest.raises(ValueError, match="out must be"):
        api.combine(recv, h, w, out=torch.empty((c.T, c.H), dtype=torch.float32,
                                                device="cuda"))
    with pytest.raises(ValueError, match="contiguous"):
        api.combine(recv, h, w, out=torch.empty((c.H, c.T), **bf).t())
    with pytest.raises(ValueError, match="topk_weights"):
        api.combine(recv, h, w[:, :1].contiguous())
    with pytest.raises(ValueError, match="GPU"):
        api.combine(recv, h, w.cpu())
    with pytest.raises(ValueError, match="unknown quant"):
        api.dispatch(x, L, quant="fp16")
    with pytest.raises(ValueError, match="cap"):
        api.dispatch(x, L, recv_layout="padded")
    with pytest.raises(ValueError, match="tokens"):
        api.dispatch(x[:-1].contiguous(), L)
    with pytest.raises(ValueError):                     # E beyond the supported 4096
        api.get_dispatch_layout(idx, 5000)

    ce = W.random_expert_choice(7, 50, 64, 4, 8, p_empty=0.0, hot=0)
    xe, te, we = G.dev(ce.x), G.dev(ce.token_indices), G.dev(ce.weights)
    with pytest.raises(ValueError, match="weights"):
        api.dispatch_expert_choice(xe, te, we[:, :4].contiguous())
    recv_e, he = api.dispatch_expert_choice(xe, te, we)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="out must be"):
        api.combine_expert_choice(recv_e, he, out=torch.empty((ce.T + 1, ce.H), **bf))
    with pytest.raises(ValueError, match="handle's weights"):
        api.combine_expert_choice(recv_e[:2].contiguous(), he)


@pytest.mark.parametrize("quant", ["fp8_e4m3_g128", "bf16"])
def test_low_latency_pair(quant):
    """low_latency_dispatch / low_latency_combine with the pages' arguments:
    the decode shape class (T = 96 tokens, capacity 16 with overflow)."""
    c = W.random_token_choice(8, 96, 512, 32, 6, p_pad=0.1, p_invalid=0.0, p_dup=0.05)
    x, idx, w = G.dev(c.x), G.dev(c.topk_idx), G.dev(c.topk_weights)
    cap = 16
    recv, scales, h = api.low_latency_dispatch(x, idx, cap, c.E, quant=quant)
    assert recv.shape[:2] == (c.E, cap)
    s_ref, _, nd_ref = oracle.slots(c.topk_idx, c.E, True, cap)
    rows = c.E * cap
    torch.cuda.synchronize()
    assert np.array_equal(G.host(h.slot), s_ref)
    assert int(G.host(h.num_dropped)[0]) == nd_ref
    assert np.array_equal(G.host(h.recv_count), np.minimum(oracle.layout(c.topk_idx, c.E)["counts"], cap))
    m = _written(s_ref, rows)
    if quant == "bf16":
        y = oracle.dispatch_bf16(c.x, s_ref, rows)
        assert np.array_equal(G.host(recv).reshape(rows, -1)[m], y[m])
        y_d = recv
    else:
        q, s = oracle.dispatch_fp8(c.x, s_ref, rows)
        assert scales.shape[:2] == (c.E, cap)
        assert np.array_equal(recv.view(torch.uint8).reshape(rows, -1).cpu().numpy()[m], q[m])
        assert np.array_equal(scales.reshape(rows, -1).cpu().numpy()[m].view(np.uint32),
                              s[m].view(np.uint32))
        # identity experts on the dequantised rows, built on the host
        deq = (np.vectorize(oracle.e4m3_to_f32)(q).astype(np.float64)
               * np.repeat(s.astype(np.float64), 128, axis=1))
        y = oracle.bf16_from_f64(deq.reshape(-1)).reshape(rows, -1)
        y_d = G.dev(y).view(c.E, cap, -1)
    out = api.low_latency_combine(y_d, idx, w, h)
    torch.cuda.synchronize()
    G.assert_combine_close(G.host(out), oracle.combine(y, s_ref, c.topk_weights))
    with pytest.raises(ValueError, match="handle"):
        api.low_latency_combine(y_d, idx[:, :2].contiguous(), w, h)


def test_rank_share_through_the_front_end():
    """pack_by_rank -> receive (the receiver's scatter with E/R experts) ->
    identity experts -> combine_partial -> combine_ranks, against the oracle
    at every step; then the same with unit weights, exactly bf16(m x)."""
    c, x, idx, w = _tc(40, T=500, H=256, E=32, K=6)
    R = 4
    per = c.E // R
    pk = api.pack_by_rank(x, idx, c.E, R, topk_weights=w)
    torch.cuda.synchronize()
    ref = oracle.rank_pack(c.x, c.topk_idx, c.topk_weights, c.E, R)
    S = int(ref["rank_offsets"][R])
    assert np.array_equal(G.host(pk.rank_offsets), ref["rank_offsets"])
    assert np.array_equal(G.host(pk.num_tokens_per_rank), np.diff(ref["rank_offsets"]))
    assert np.array_equal(G.host(pk.pack_pos), ref["pack_pos"])
    assert np.array_equal(G.host(pk.send_x[:S]), ref["send_x"][:S])
    assert np.array_equal(G.host(pk.send_idx[:S]), ref["send_idx"][:S])
    assert np.array_equal(G.host(pk.send_w[:S]), ref["send_w"][:S])
    assert int(G.host(pk.num_dropped)[0]) == 0 and pk.experts_per_rank == per
    L, recv, scales, h = api.receive(pk.send_x[:S].contiguous(), pk.send_idx[:S].contiguous(), per)
    part = api.combine_partial(recv, h, pk.send_w[:S].contiguous())
    out = api.combine_ranks(part, pk)
    torch.cuda.synchronize()
    s_ref, _, _ = oracle.slots(ref["send_idx"][:S], per, False, S * c.K)
    assert scales is None and np.array_equal(G.host(h.slot), s_ref)
    y = oracle.dispatch_bf16(ref["send_x"][:S], s_ref, S * c.K)
    part_ref = oracle.combine_partial(y, s_ref, ref["send_w"][:S])
    G.assert_f32_close(G.host(part), part_ref)
    G.assert_combine_close(G.host(out), oracle.combine_ranks(part_ref, ref["pack_pos"]))
    # unit weights: the pack sends ones, the round trip is exact
    pk1 = api.pack_by_rank(x, idx, c.E, R)
    _, recv1, _, h1 = api.receive(pk1.send_x[:S].contiguous(), pk1.send_idx[:S].contiguous(), per)
    out1 = api.combine_ranks(api.combine_partial(recv1, h1, pk1.send_w[:S].contiguous()), pk1)
    torch.cuda.synchronize()
    m = ((c.topk_idx >= 0) & (c.topk_idx < c.E)).sum(axis=1)
    assert np.array_equal(G.host(out1), brute.multiplicity_times_x(c.x, m))


def test_rank_share_argument_checks():
    c, x, idx, w = _tc(41, T=50, H=64, E=8, K=3)
    with pytest.raises(ValueError):
        api.pack_by_rank(x, idx, c.E, 3)                      # E % R != 0
    with pytest.raises(ValueError):
        api.pack_by_rank(x[:10], idx, c.E, 4)                 # token counts disagree
    with pytest.raises(ValueError):
        api.pack_by_rank(x, idx, c.E, 4, topk_weights=w[:, :2].contiguous())
    pk = api.pack_by_rank(x, idx, c.E, 4)
    with pytest.raises(ValueError):
        api.combine_ranks(torch.zeros((4, 64), dtype=torch.bfloat16, device=G.DEV), pk)
    _, recv, _, h = api.receive(pk.send_x, pk.send_idx, 2)
    with pytest.raises(ValueError):
        api.combine_partial(recv, h, torch.ones((3, 3), dtype=torch.float32, device=G.DEV))
    torch.cuda.synchronize()
