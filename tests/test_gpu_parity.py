"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for layout, slots, recv_src, dispatched bf16 rows and fp8
codes/scales, inverse maps and counters; combine within
|gpu - oracle| <= 2^-7 |oracle| + 1e-3 per element.  Every input comes from
the seeded generator or from the oracle, never from the GPU path.  Small
cases span several chunks/tiles and ragged tails; the five named workloads
run at full size in the same launch configuration the benchmark uses, with
every token and every kept receive row compared against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import brute
import golden_io
import gpu_util as G
import oracle
from combine_get_dispatch_04_amd import workloads as W

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- layout
LAYOUT_CASES = [
    # T, K, E, R, p_pad, p_invalid
    (1, 1, 1, 1, 0.0, 0.0),
    (5, 3, 7, 7, 0.3, 0.2),
    (128, 2, 8, 2, 0.0, 0.0),
    (1000, 8, 256, 8, 0.1, 0.01),
    (1025, 6, 64, 64, 0.2, 0.05),
    (3001, 8, 256, 1, 0.05, 0.0),
    (777, 40, 96, 96, 0.3, 0.0),         # K > 32
    (700, 4, 1024, 128, 0.1, 0.01),      # R > 64 path
    (300, 3, 4096, 4, 0.0, 0.02),        # largest E
    (9000, 1, 2, 1, 0.5, 0.1),
    (20000, 16, 384, 8, 0.15, 0.0),      # many chunks, every scan column in one LDS tile
    (6000, 8, 4096, 16, 0.1, 0.01),      # many chunks and E = 4096: the scan takes several tiles
]


@pytest.mark.parametrize("T,K,E,R,pp,pi", LAYOUT_CASES)
def test_layout_parity(T, K, E, R, pp, pi):
    _announce(f"layout T={T} K={K} E={E} R={R}")
    c = W.random_token_choice(T * 7 + K, T, 8, E, K, p_pad=pp, p_invalid=pi, p_dup=0.1)
    L = G.layout(G.dev(c.topk_idx), E, R)
    torch.cuda.synchronize()
    ref = oracle.layout(c.topk_idx, E, R)
    for key in ("counts", "offsets", "tokens_per_rank", "is_token_in_rank"):
        assert np.array_equal(G.host(L[key]), ref[key]), key
    assert int(G.host(L["num_invalid"])[0]) == ref["num_invalid"]


def test_layout_without_rank_outputs_and_empty():
    _announce("layout NULL rank outputs, T=0")
    c = W.random_token_choice(3, 50, 8, 16, 4)
    L = G.layout(G.dev(c.topk_idx), 16, 4, with_rank=False)
    torch.cuda.synchronize()
    ref = oracle.layout(c.topk_idx, 16, 4)
    assert np.array_equal(G.host(L["offsets"]), ref["offsets"])
    idx0 = torch.empty((0, 4), dtype=torch.int32, device=G.DEV)
    L = G.layout(idx0, 16, 4)
    torch.cuda.synchronize()
    assert (G.host(L["counts"]) == 0).all() and (G.host(L["offsets"]) == 0).all()
    assert (G.host(L["tokens_per_rank"]) == 0).all() and int(G.host(L["num_invalid"])[0]) == 0


# ---------------------------------------------------------------- dispatch (bf16)
def _check_dispatch(c, padded, cap, recv, slot, src, nd, fp8=False, sc=None):
    rows = c.E * cap if padded else cap
    s_ref, src_ref, nd_ref = oracle.slots(c.topk_idx, c.E, padded, cap)
    s = G.host(slot)
    assert np.array_equal(s, s_ref)
    assert int(G.host(nd)[0]) == nd_ref
    written = np.zeros(rows, bool)
    written[s_ref[s_ref >= 0]] = True
    gsrc = G.host(src)[:rows]
    assert np.array_equal(gsrc[written], src_ref[written])
    assert (gsrc[~written] == -2).all()                      # nothing else written
    r = G.host(recv)
    if fp8:
        q_ref, sc_ref = oracle.dispatch_fp8(c.x, s_ref, rows)
        assert np.array_equal(r[written], q_ref[written])
        assert np.array_equal(G.host(sc)[written].view(np.uint32), sc_ref[written].view(np.uint32))
        assert (r[~written] == G.SENT8).all()
    else:
        ref = oracle.dispatch_bf16(c.x, s_ref, rows)
        assert np.array_equal(r[written], ref[written])
        assert (r[~written] == G.SENT16).all()


DISPATCH_CASES = [
    # T, H, E, K, layout, cap
    (1, 8, 1, 1, "contiguous", None),
    (37, 24, 5, 3, "contiguous", None),
    (513, 520, 16, 4, "contiguous", None),          # ragged rows: 65 pieces
    (300, 2056, 32, 6, "contiguous", None),         # 257 pieces, two row segments
    (1000, 7168, 256, 8, "contiguous", None),
    (400, 96, 12, 5, "contiguous", "short"),        # receive buffer smaller than N
    (257, 128, 9, 4, "padded", 3),                  # capacity overflow
    (128, 256, 8, 8, "padded", 200),
    (2000, 64, 100, 40, "contiguous", None),        # K > 32
    (5000, 16, 2, 1, "padded", 1000),
]


@pytest.mark.parametrize("T,H,E,K,lay,cap", DISPATCH_CASES)
def test_dispatch_bf16_parity(T, H, E, K, lay, cap):
    _announce(f"dispatch bf16 T={T} H={H} E={E} K={K} {lay} cap={cap}")
    c = W.random_token_choice(T + H + E, T, H, E, K, p_pad=0.15, p_invalid=0.03, p_dup=0.15)
    padded = lay == "padded"
    if cap == "short":
        N = int(((c.topk_idx >= 0) & (c.topk_idx < E)).sum())
        cap = N - 17
    elif cap is None:
        cap = T * K
    x_d, idx_d = G.dev(c.x), G.dev(c.topk_idx)
    L = G.layout(idx_d, E)
    recv, _, slot, src, nd = G.dispatch(x_d, idx_d, E, L, padded, cap)
    torch.cuda.synchronize()
    _check_dispatch(c, padded, cap, recv, slot, src, nd)


def test_dispatch_empty_and_all_padding():
    _announce("dispatch T=0 and all -1")
    idx0 = torch.empty((0, 3), dtype=torch.int32, device=G.DEV)
    x0 = torch.empty((0, 64), dtype=torch.bfloat16, device=G.DEV)
    L = G.layout(idx0, 4)
    recv, _, slot, src, nd = G.dispatch(x0, idx0, 4, L, False, 0)
    torch.cuda.synchronize()
    assert int(G.host(nd)[0]) == 0
    c = W.random_token_choice(1, 60, 32, 4, 3, p_pad=1.0)
    x_d, idx_d = G.dev(c.x), G.dev(c.topk_idx)
    L = G.layout(idx_d, 4)
    recv, _, slot, src, nd = G.dispatch(x_d, idx_d, 4, L, True, 5)
    torch.cuda.synchronize()
    assert (G.host(slot) == -1).all() and int(G.host(nd)[0]) == 0
    assert (G.host(recv) == G.SENT16).all()


# ---------------------------------------------------------------- dispatch (fp8)
@pytest.mark.parametrize("T,H,E,K,lay,cap", [
    (3, 128, 2, 1, "contiguous", None),
    (77, 384, 10, 3, "padded", 4),
    (300, 7168, 64, 8, "contiguous", None),
    (129, 1280, 256, 8, "padded", 128),     # 10 groups per row
])
def test_dispatch_fp8_parity(T, H, E, K, lay, cap):
    _announce(f"dispatch fp8 T={T} H={H} E={E} K={K} {lay}")
    c = W.random_token_choice(T + 3 * H, T, H, E, K, p_pad=0.1, p_invalid=0.02)
    xf = W.bf16_to_f32(c.x).copy()
    xf[0, :128] = 0.0                                  # an all-zero group
    if T > 2:
        xf[1, :128] *= 2.0 ** -30                      # tiny values, subnormal codes
        xf[2, 128 % H:128 % H + 128] *= 1e4 if H > 128 else 1.0
    c.x = W.bf16_bits(xf)
    padded = lay == "padded"
    cap = T * K if cap is None else cap
    x_d, idx_d = G.dev(c.x), G.dev(c.topk_idx)
    L = G.layout(idx_d, E)
    recv, sc, slot, src, nd = G.dispatch(x_d, idx_d, E, L, padded, cap, fp8=True)
    torch.cuda.synchronize()
    _check_dispatch(c, padded, cap, recv, slot, src, nd, fp8=True, sc=sc)


def test_dispatch_fp8_golden_group():
    """The hand-derived ties/subnormal/sign cases, through the GPU encoder."""
    _announce("fp8 golden group")
    g = golden_io.read_kv("fp8_group_small.txt")
    H = g["H"][0]
    xv = np.zeros(H, np.float32)
    head = np.array(g["x_group0_head"], np.float32)
    xv[:head.size] = head
    xv[128 + 5] = -0.0
    x = W.bf16_bits(xv[None, :])
    idx = np.array([[0, 1]], np.int32)
    x_d, idx_d = G.dev(x), G.dev(idx)
    L = G.layout(idx_d, 2)
    recv, sc, slot, src, nd = G.dispatch(x_d, idx_d, 2, L, True, 1, fp8=True)
    torch.cuda.synchronize()
    q = G.host(recv)
    for r in (0, 1):
        assert q[r, :head.size].tolist() == g["q_group0_head"]
        assert (q[r, head.size:] == 0).all()
        assert G.host(sc)[r].tolist() == g["scales"]


def test_fp8_every_e4m3_boundary():
    """A row built so that x / s lands exactly on every e4m3 value, every
    midpoint, and one bf16 step either side (s = 2^-4, so the division is an
    exact scaling): the GPU codes must equal the oracle's."""
    _announce("fp8 boundaries")
    tab = brute.e4m3_table()
    pos = np.sort(tab[:127][~np.isnan(tab[:127])])
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([pos, mids]).astype(np.float32)
    # keep only values that bf16 holds exactly at scale 2^-4, then 1-ulp-of-bf16 neighbours
    scale = np.float32(2.0 ** -4)
    xs = vals * scale
    xb = W.bf16_bits(xs)
    ok = W.bf16_to_f32(xb) == xs
    xs = xs[ok]
    nb_up = W.bf16_to_f32(W.bf16_bits(xs) + 1)
    nb_dn = W.bf16_to_f32(np.maximum(W.bf16_bits(xs).astype(np.int32) - 1, 0).astype(np.uint16))
    allv = np.concatenate([xs, nb_up, nb_dn, -xs])
    # 127 values per group plus the amax 448*scale as channel 0 of every group
    per = 127
    ngroups = (allv.size + per - 1) // per
    H = 128 * ngroups
    row = np.zeros(H, np.float32)
    for g in range(ngroups):
        chunk = allv[g * per:(g + 1) * per]
        row[128 * g] = 448.0 * scale
        row[128 * g + 1:128 * g + 1 + chunk.size] = np.minimum(np.abs(chunk), 448 * scale) * np.sign(chunk)
    x = W.bf16_bits(row[None, :])
    idx = np.zeros((1, 1), np.int32)
    x_d, idx_d = G.dev(x), G.dev(idx)
    L = G.layout(idx_d, 1)
    recv, sc, slot, src, nd = G.dispatch(x_d, idx_d, 1, L, False, 1, fp8=True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.dispatch_fp8(x, np.zeros((1, 1), np.int32), 1)
    assert np.array_equal(G.host(recv), q_ref)
    assert np.array_equal(G.host(sc), s_ref)


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("T,H,E,K,weighted", [
    (1, 8, 1, 1, True), (50, 64, 6, 3, True), (513, 520, 16, 4, False),
    (300, 2056, 32, 6, True), (1000, 7168, 256, 8, True), (2000, 64, 100, 40, True),
    # K >= 12: 2 pieces per thread, 4 rows per round (a ragged last round at 13)
    (300, 7168, 64, 16, True), (257, 520, 20, 13, False), (100, 2056, 32, 12, True),
    # T >= 1024 and K < 12: one row per round; 7 pieces per thread at H = 7168
    # (the prefill instantiation), 4 at a ragged 897-piece row
    (1024, 7168, 256, 8, True), (1500, 7168, 64, 8, False), (1031, 7176, 40, 8, True),
])
def test_combine_parity(T, H, E, K, weighted):
    _announce(f"combine T={T} H={H} K={K} w={weighted}")
    c = W.random_token_choice(5 * T + H, T, H, E, K, p_pad=0.2, p_invalid=0.05, p_dup=0.2)
    s_ref, _, _ = oracle.slots(c.topk_idx, E, False, T * K)
    rng = np.random.default_rng(T + K)
    y = W.bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    w = (rng.standard_normal((T, K)) * 2).astype(np.float32) if weighted else None
    out = G.combine(G.dev(y), G.dev(s_ref), G.dev(w) if w is not None else None)
    torch.cuda.synchronize()
    G.assert_combine_close(G.host(out), oracle.combine(y, s_ref, w))


def test_combine_unit_weights_round_trip_exact():
    """dispatch then unit-weight combine = bf16(m_t * x_t), bit for bit."""
    _announce("combine round trip")
    c = W.random_token_choice(77, 900, 520, 24, 12, p_pad=0.3, p_dup=0.3)
    x_d, idx_d = G.dev(c.x), G.dev(c.topk_idx)
    L = G.layout(idx_d, c.E)
    recv, _, slot, _, _ = G.dispatch(x_d, idx_d, c.E, L)
    out = G.combine(recv, slot, None)
    torch.cuda.synchronize()
    m = (c.topk_idx >= 0).sum(axis=1)
    assert np.array_equal(G.host(out), brute.multiplicity_times_x(c.x, m))


# ---------------------------------------------------------------- expert choice
# The inverse map is built by one block from per-token expert bitmasks in
# LDS, or, when some expert lists a token twice, by the same block with
# counters and a rank sort.  That block runs inside the copy's launch when
# the T*ceil(E/64) mask words take at most 81664 bytes, in a launch of its
# own up to the device's LDS per block (160 KiB), and beyond that five
# launches do the work with the counters in the workspace.
EC_CASES = [
    # T, H, E, C, p_empty, p_invalid, hot, distinct
    (1, 8, 1, 1, 0.0, 0.0, 0, False),
    (10, 24, 3, 4, 0.2, 0.1, 0, False),
    (500, 520, 16, 64, 0.1, 0.02, 5, False),
    (300, 4096, 64, 40, 0.0, 0.0, 40, False),    # tokens picked by all 64 experts
    (50, 64, 1200, 2, 0.0, 0.0, 1, False),       # one token picked 1200 times (> one sort tile)
    (0, 16, 3, 5, 0.0, 0.0, 0, False),           # no tokens: every entry is -1
    (0, 16, 3, 5, 0.0, 0.3, 0, False),           # no tokens, some entries invalid
    (500, 520, 16, 64, 0.1, 0.05, 5, True),      # bitmask path, empty and invalid entries
    (64, 40, 64, 64, 0.0, 0.0, 64, True),        # every expert picks every token (bit 63 used)
    (300, 96, 100, 20, 0.05, 0.0, 7, True),      # two mask words per token
    (64, 8, 130, 8, 0.0, 0.0, 3, True),          # three mask words, hot tokens in all of them
    (1, 8, 5, 1, 0.0, 0.0, 1, True),             # one token, every expert
    (5000, 8, 32, 200, 0.0, 0.0, 0, False),      # duplicate path at a larger T
    (10200, 8, 8, 1000, 0.1, 0.01, 3, True),     # 81600 B of masks: inside the copy's launch
    (13000, 8, 8, 1000, 0.1, 0.01, 3, True),     # 104000 B: a launch of its own
    (20000, 8, 8, 1000, 0.1, 0.01, 3, True),     # 160000 B: a launch of its own
    (20000, 8, 8, 1000, 0.0, 0.0, 0, False),     # 160000 B with duplicates
    (30000, 8, 8, 512, 0.1, 0.01, 3, True),      # 240000 B: five launches
    (30000, 16, 4, 600, 0.0, 0.0, 2, False),     # five launches with duplicates
]


@pytest.mark.parametrize("T,H,E,C,pe,pi,hot,distinct", EC_CASES)
def test_expert_choice_parity(T, H, E, C, pe, pi, hot, distinct):
    _announce(f"ec T={T} H={H} E={E} C={C} hot={hot} distinct={distinct}")
    c = W.random_expert_choice(T + E * C, T, H, E, C, p_empty=pe, p_invalid=pi, hot=hot,
                               distinct=distinct)
    x_d, ti_d = G.dev(c.x), G.dev(c.token_indices)
    recv, off, ent, ninv = G.ec_dispatch(x_d, ti_d)
    torch.cuda.synchronize()
    off_ref, ent_ref = oracle.ec_invert(c.token_indices, T)
    assert np.array_equal(G.host(off), off_ref)
    n = int(off_ref[-1])
    assert np.array_equal(G.host(ent)[:n], ent_ref[:n])
    sentinel = np.full((E, C, H), G.SENT16, np.uint16)
    recv_ref, ninv_ref = oracle.ec_dispatch(c.x, c.token_indices, sentinel)
    assert int(G.host(ninv)[0]) == ninv_ref
    assert np.array_equal(G.host(recv), recv_ref)
    rng = np.random.default_rng(E + C)
    y = W.bf16_bits(rng.standard_normal((E, C, H), dtype=np.float32))
    out = G.ec_combine(G.dev(y), G.dev(c.weights), off, ent, T)
    torch.cuda.synchronize()
    if T:
        G.assert_combine_close(G.host(out), oracle.ec_combine(y, c.weights, c.token_indices, T))


def test_expert_choice_round_trip_exact():
    _announce("ec round trip")
    c = W.random_expert_choice(5, 700, 264, 48, 30, p_empty=0.1, hot=10)
    x_d, ti_d = G.dev(c.x), G.dev(c.token_indices)
    recv, off, ent, _ = G.ec_dispatch(x_d, ti_d)
    ones = torch.ones((c.E, c.C), dtype=torch.float32, device=G.DEV)
    # -1 entries leave sentinel rows, but no token's entry list names them
    out = G.ec_combine(recv, ones, off, ent, c.T)
    torch.cuda.synchronize()
    flat = c.token_indices.ravel()
    m = np.bincount(flat[flat >= 0], minlength=c.T)
    assert (m == 0).any() and (m > 32).any()
    assert np.array_equal(G.host(out), brute.multiplicity_times_x(c.x, m))


# ---------------------------------------------------------------- the named workloads
def _token_choice_full(c):
    """A named workload at full size, launched as the benchmark launches it:
    layout (R = 8), slots, every kept receive row (codes and scales for fp8)
    and the weighted and unit-weight combine of every token against the
    oracle."""
    padded = c.layout == "padded"
    fp8 = c.quant == "fp8_e4m3_g128"
    cap = c.cap if padded else c.T * c.K
    rows = c.E * cap if padded else cap
    x_d, idx_d = G.dev(c.x), G.dev(c.topk_idx)
    L = G.layout(idx_d, c.E, 8)
    recv, sc, slot, src, nd = G.dispatch(x_d, idx_d, c.E, L, padded, cap, fp8=fp8,
                                         sentinel=not (c.T * c.K * c.H > 1e8))
    torch.cuda.synchronize()
    ref = oracle.layout(c.topk_idx, c.E, 8)
    for key in ("counts", "offsets", "tokens_per_rank", "is_token_in_rank"):
        assert np.array_equal(G.host(L[key]), ref[key]), key
    s_ref, src_ref, nd_ref = oracle.slots(c.topk_idx, c.E, padded, cap)
    assert np.array_equal(G.host(slot), s_ref)
    assert int(G.host(nd)[0]) == nd_ref
    wr = s_ref[s_ref >= 0]
    assert np.array_equal(G.host(src)[wr], src_ref[wr])
    if fp8:
        q_ref, sc_ref = oracle.dispatch_fp8(c.x, s_ref, rows)
        assert np.array_equal(G.host(recv[torch.from_numpy(wr).to(G.DEV).long()]), q_ref[wr])
        assert np.array_equal(G.host(sc)[wr], sc_ref[wr])
        # y = dequantised rows (identity expert), built on the host from the oracle's codes
        tab = brute.e4m3_table().astype(np.float32)
        y = np.zeros((rows, c.H), np.uint16)
        deq = tab[q_ref[wr]] * np.repeat(sc_ref[wr], 128, axis=1)
        y[wr] = W.bf16_bits(deq)
        y_d = G.dev(y)
    else:
        # every kept receive row against the oracle's own copy (compared on
        # the GPU: the large workload's rows are 3.2 GB)
        y = oracle.dispatch_bf16(c.x, s_ref, rows)
        y_d = G.dev(y)
        sel = torch.from_numpy(wr.astype(np.int64)).to(G.DEV)
        for lo in range(0, sel.numel(), 8192):
            s_ = sel[lo:lo + 8192]
            assert torch.equal(recv.view(torch.int16)[s_], y_d.view(torch.int16)[s_]), lo
    # combine of every token from the oracle-built y, with the routing
    # weights and with unit weights
    del recv
    w = c.topk_weights
    out = G.combine(y_d, G.dev(s_ref), G.dev(w))
    out1 = G.combine(y_d, G.dev(s_ref), None)
    torch.cuda.synchronize()
    G.assert_combine_close(G.host(out), oracle.combine(y, s_ref, w), c.name)
    G.assert_combine_close(G.host(out1), oracle.combine(y, s_ref, None), c.name + " unit")
    if not fp8:
        # size-free exact pin: unit weights over y = dispatch(x) gives bf16(m x)
        m = torch.from_numpy((s_ref >= 0).sum(axis=1).astype(np.float32)).to(G.DEV)
        prod = x_d.float() * m[:, None]
        exp = torch.where(prod == 0, 0.0, prod).to(torch.bfloat16)      # sums start from +0
        assert torch.equal(out1.view(torch.int16), exp.view(torch.int16))


def test_workload_toy():
    _announce("workload toy")
    _token_choice_full(W.toy())


def test_workload_decode_fp8_padded():
    _announce("workload decode fp8 padded")
    _token_choice_full(W.decode())


def test_workload_prefill():
    _announce("workload prefill")
    _token_choice_full(W.prefill())


def test_workload_large_padded():
    _announce("workload large -1 padded")
    _token_choice_full(W.large_padded())


def test_workload_expert_choice():
    _announce("workload expert choice")
    c = W.expert_choice()
    x_d, ti_d = G.dev(c.x), G.dev(c.token_indices)
    recv, off, ent, ninv = G.ec_dispatch(x_d, ti_d)
    torch.cuda.synchronize()
    off_ref, ent_ref = oracle.ec_invert(c.token_indices, c.T)
    assert np.array_equal(G.host(off), off_ref)
    assert np.array_equal(G.host(ent), ent_ref)
    recv_ref, ninv_ref = oracle.ec_dispatch(c.x, c.token_indices)
    assert int(G.host(ninv)[0]) == ninv_ref == 0
    assert np.array_equal(G.host(recv), recv_ref)
    y_d = G.dev(recv_ref)
    out = G.ec_combine(y_d, G.dev(c.weights), off, ent, c.T)
    ones = torch.ones((c.E, c.C), dtype=torch.float32, device=G.DEV)
    out1 = G.ec_combine(y_d, ones, off, ent, c.T)
    torch.cuda.synchronize()
    G.assert_combine_close(G.host(out), oracle.ec_combine(recv_ref, c.weights, c.token_indices, c.T))
    flat = c.token_indices.ravel()
    m = np.bincount(flat, minlength=c.T)
    assert np.array_equal(G.host(out1), brute.multiplicity_times_x(c.x, m))


def test_determinism_prefill():
    _announce("determinism prefill")
    c = W.prefill()
    x_d, idx_d = G.dev(c.x), G.dev(c.topk_idx)
    w_d = G.dev(c.topk_weights)
    res = []
    for _ in range(2):
        L = G.layout(idx_d, c.E)
        recv, _, slot, src, _ = G.dispatch(x_d, idx_d, c.E, L, sentinel=False)
        out = G.combine(recv, slot, w_d)
        torch.cuda.synchronize()
        res.append((slot.clone(), out.view(torch.int16).clone(),
                    recv.view(torch.int16)[:32768].clone()))
        del recv
    for a, b in zip(*res):
        assert torch.equal(a, b)
