"""Pins for the oracle's token-choice path: layout, slots, bf16/fp8 dispatch,
combine.  Each pin is independent of oracle.c: hand-derived fixtures, numpy
brute force, textbook special cases, closed forms and invariants."""
import numpy as np
import pytest
import torch

import brute
import golden_io
import oracle
from combine_get_dispatch_04_amd import workloads as W


# ------------------------------------------------------------------ fixture
def _fixture():
    g = golden_io.read_kv("token_choice_small.txt")
    T, K, E, R = g["T"][0], g["K"][0], g["E"][0], g["R"][0]
    idx = np.array(g["topk_idx"], np.int32).reshape(T, K)
    return g, T, K, E, R, idx


def test_golden_layout():
    g, T, K, E, R, idx = _fixture()
    L = oracle.layout(idx, E, R)
    assert L["counts"].tolist() == g["counts"]
    assert L["offsets"].tolist() == g["offsets"]
    assert L["num_invalid"] == g["num_invalid"][0]
    assert L["is_token_in_rank"].ravel().tolist() == g["is_token_in_rank"]
    assert L["tokens_per_rank"].tolist() == g["tokens_per_rank"]


def test_golden_slots():
    g, T, K, E, R, idx = _fixture()
    slot, src, nd = oracle.slots(idx, E, False, T * K)
    assert slot.ravel().tolist() == g["slot_contiguous"] and nd == 0
    assert src[:7].tolist() == g["recv_src_contiguous"]
    slot, src, nd = oracle.slots(idx, E, True, 2)
    assert slot.ravel().tolist() == g["slot_padded_cap2"] and nd == g["dropped_padded_cap2"][0]
    slot, src, nd = oracle.slots(idx, E, False, 5)
    assert slot.ravel().tolist() == g["slot_contiguous_rows5"]
    assert nd == g["dropped_contiguous_rows5"][0]


def test_golden_combine():
    g, T, K, E, R, idx = _fixture()
    H = 16
    xv = np.array(g["x_row_values"], np.float32)
    x = W.bf16_bits(np.repeat(xv[:, None], H, axis=1))
    slot, _, _ = oracle.slots(idx, E, False, T * K)
    y = oracle.dispatch_bf16(x, slot, T * K)
    out = oracle.combine(y, slot, None)
    assert (out == np.array(g["out_unit_bf16"], np.uint16)[:, None]).all()
    w = np.array(g["weights"], np.float32).reshape(T, K)
    out = oracle.combine(y, slot, w)
    assert (out == np.array(g["out_weighted_bf16"], np.uint16)[:, None]).all()


# ------------------------------------------------------------------ brute force
CASES = [(seed, T, K, E) for seed, (T, K, E) in enumerate(
    [(1, 1, 1), (7, 3, 5), (16, 2, 4), (33, 6, 16), (64, 4, 3), (50, 8, 64), (0, 4, 8), (5, 1, 2)])]


@pytest.mark.parametrize("seed,T,K,E", CASES)
def test_layout_vs_brute(seed, T, K, E):
    for R in [r for r in (1, 2, E) if E % r == 0]:
        c = W.random_token_choice(seed, T, 8, E, K, p_pad=0.2, p_invalid=0.1, p_dup=0.2)
        a = oracle.layout(c.topk_idx, E, R)
        b = brute.layout(c.topk_idx, E, R)
        for key in ("counts", "offsets", "tokens_per_rank", "is_token_in_rank"):
            assert np.array_equal(a[key], b[key]), key
        assert a["num_invalid"] == b["num_invalid"]


@pytest.mark.parametrize("seed,T,K,E", CASES)
def test_slots_vs_brute(seed, T, K, E):
    c = W.random_token_choice(seed, T, 8, E, K, p_pad=0.2, p_invalid=0.1, p_dup=0.3)
    N = int(((c.topk_idx >= 0) & (c.topk_idx < E)).sum())
    for padded, cap in [(False, T * K), (False, max(N - 3, 0)), (True, 1), (True, 2), (True, T * K)]:
        s1, _, d1 = oracle.slots(c.topk_idx, E, padded, cap)
        s2, d2 = brute.slots(c.topk_idx, E, padded, cap)
        assert np.array_equal(s1, s2), (padded, cap)
        assert d1 == d2


def test_k1_slots_are_inverse_stable_argsort():
    """Textbook special case: with K = 1 and no padding, the contiguous slot of
    token t is its position in a stable sort of the expert ids."""
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 13, size=(500, 1)).astype(np.int32)
    slot, _, _ = oracle.slots(idx, 13, False, 500)
    order = np.argsort(idx[:, 0], kind="stable")
    inv = np.empty(500, np.int64)
    inv[order] = np.arange(500)
    assert np.array_equal(slot[:, 0], inv)


# ------------------------------------------------------------------ invariants
def _check_slot_invariants(idx, E, slot, src, counts, offsets):
    valid = (idx >= 0) & (idx < E)
    N = int(valid.sum())
    assert counts.sum() == N
    assert offsets[-1] == N and np.array_equal(np.diff(offsets), counts)
    s = slot[valid]
    assert (slot[~valid] == -1).all()
    assert np.array_equal(np.sort(s), np.arange(N))            # bijection onto [0, N)
    e_of_row = np.repeat(np.arange(E), counts)
    t_of = np.nonzero(valid)[0]
    assert np.array_equal(e_of_row[s], idx[valid])             # row lies in its expert's block
    assert np.array_equal(src[s], t_of)
    for e in range(E):                                          # ascending token order per expert
        blk = src[offsets[e]:offsets[e + 1]]
        assert (np.diff(blk) >= 0).all()


@pytest.mark.parametrize("make", [W.toy, W.decode, W.prefill])
def test_slot_invariants_on_workloads(make):
    c = make()
    L = oracle.layout(c.topk_idx, c.E)
    slot, src, nd = oracle.slots(c.topk_idx, c.E, False, c.T * c.K)
    assert nd == 0 and L["num_invalid"] == 0
    _check_slot_invariants(c.topk_idx, c.E, slot, src, L["counts"], L["offsets"])


def test_prefill_routing_statistics():
    """The skewed workload's routing matches its recipe (recorded statistics)."""
    c = W.prefill()
    L = oracle.layout(c.topk_idx, c.E)
    assert L["offsets"][-1] == 4096 * 8
    # Zipf(1.2) bias with coefficient 2 concentrates top-8 on a few dozen experts;
    # the hottest is chosen by (almost) every token
    assert 16 <= (L["counts"] > 0).sum() <= 64
    assert L["counts"].max() >= 4000
    assert (np.diff(np.sort(c.topk_idx, axis=1), axis=1) > 0).all()   # distinct experts per token


def test_padded_invariants():
    c = W.random_token_choice(9, 300, 8, 16, 6, p_pad=0.1, p_dup=0.1)
    cap = 40
    slot, src, nd = oracle.slots(c.topk_idx, c.E, True, cap)
    L = oracle.layout(c.topk_idx, c.E)
    valid = (c.topk_idx >= 0)
    kept = slot >= 0
    assert nd == int(np.maximum(L["counts"] - cap, 0).sum())
    assert np.array_equal(slot[kept] // cap, c.topk_idx[kept])
    for e in range(c.E):
        rows = np.sort(slot[kept & (c.topk_idx == e)]) - e * cap
        assert np.array_equal(rows, np.arange(min(L["counts"][e], cap)))
    assert (kept <= valid).all()


# ------------------------------------------------------------------ dispatch
def test_dispatch_bf16_closed_form():
    c = W.random_token_choice(4, 97, 72, 9, 5, p_pad=0.2, p_dup=0.2)
    slot, _, _ = oracle.slots(c.topk_idx, c.E, False, c.T * c.K)
    recv = oracle.dispatch_bf16(c.x, slot, c.T * c.K)
    for t in range(c.T):
        for k in range(c.K):
            if slot[t, k] >= 0:
                assert np.array_equal(recv[slot[t, k]], c.x[t])


def test_fp8_golden_group():
    g = golden_io.read_kv("fp8_group_small.txt")
    H = g["H"][0]
    xv = np.zeros(H, np.float32)
    head = np.array(g["x_group0_head"], np.float32)
    xv[:head.size] = head
    xv[128 + 5] = -0.0
    x = W.bf16_bits(xv[None, :])
    assert np.array_equal(W.bf16_to_f32(x)[0], xv)      # all fixture values are bf16 values
    slot = np.array([[0, 1]], np.int32)
    q, s = oracle.dispatch_fp8(x, slot, 2)
    for r in (0, 1):
        assert q[r, :head.size].tolist() == g["q_group0_head"]
        assert (q[r, head.size:] == 0).all()
        assert s[r].tolist() == g["scales"]


def test_fp8_vs_brute_rows():
    c = W.random_token_choice(12, 6, 512, 4, 2, p_pad=0.0)
    # make one group all zero and one group tiny
    xf = W.bf16_to_f32(c.x).copy()
    xf[1, 128:256] = 0.0
    xf[2, 0:128] *= 2.0 ** -20
    xf[3, 256:384] = np.where(np.arange(128) % 2 == 0, -0.0, 0.0)
    x = W.bf16_bits(xf)
    slot = np.arange(c.T, dtype=np.int32)[:, None]
    q, s = oracle.dispatch_fp8(x, slot, c.T)
    for t in range(c.T):
        qb, sb = brute.fp8_quant_token(x[t])
        assert np.array_equal(q[t], qb), t
        assert np.array_equal(s[t], sb), t


def test_fp8_closed_forms_on_decode_workload():
    """amax element -> +-448 code; zero groups -> zeros; |x - q s| within the
    e4m3 rounding bound."""
    c = W.decode()
    slot, _, _ = oracle.slots(c.topk_idx, c.E, True, c.cap)
    rows = c.E * c.cap
    q, s = oracle.dispatch_fp8(c.x, slot, rows)
    xf = W.bf16_to_f32(c.x).astype(np.float64)
    tab = brute.e4m3_table()
    for t in range(c.T):
        r = slot[t][slot[t] >= 0][0]
        for g in range(c.H // 128):
            blk = xf[t, 128 * g:128 * (g + 1)]
            a = np.abs(blk).max()
            assert s[r, g] == np.float32(np.float32(a) / np.float32(448))
            qq = q[r, 128 * g:128 * (g + 1)]
            i = int(np.argmax(np.abs(blk)))
            assert qq[i] == (0xFE if blk[i] < 0 else 0x7E)
            deq = tab[qq] * float(s[r, g])
            bound = np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * float(s[r, g])) * (1 + 2.0 ** -20)
            assert (np.abs(blk - deq) <= bound).all()
        # every kept slot of t holds the same bytes
        for k in range(c.K):
            if slot[t, k] >= 0:
                assert np.array_equal(q[slot[t, k]], q[r]) and np.array_equal(s[slot[t, k]], s[r])


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("seed,T,K,E", CASES[:6])
def test_combine_vs_brute(seed, T, K, E):
    c = W.random_token_choice(seed, T, 24, E, K, p_pad=0.2, p_invalid=0.05, p_dup=0.2)
    slot, _, _ = oracle.slots(c.topk_idx, E, False, T * K)
    rng = np.random.default_rng(seed + 100)
    y = W.bf16_bits(rng.standard_normal((max(T * K, 1), 24), dtype=np.float32))
    w = (rng.standard_normal((T, K)) * 3).astype(np.float32)
    assert np.array_equal(oracle.combine(y, slot, w), brute.combine_f64(y, slot, w))
    assert np.array_equal(oracle.combine(y, slot, None), brute.combine_f64(y, slot, None))


def test_combine_unit_weight_round_trip_is_multiplicity_times_x():
    """dispatch then combine with unit weights = bf16(m_t * x_t): every partial
    sum j*x is exact, so the only rounding is the final one.  m_t * x_t is
    formed in fp32 (exact for m_t <= 2^16) and rounded by torch's cast."""
    c = W.random_token_choice(21, 200, 64, 12, 7, p_pad=0.3, p_dup=0.4)
    c.topk_idx[:3] = -1                                   # tokens with no slot at all
    slot, _, _ = oracle.slots(c.topk_idx, c.E, False, c.T * c.K)
    y = oracle.dispatch_bf16(c.x, slot, c.T * c.K)
    out = oracle.combine(y, slot, None)
    m = (slot >= 0).sum(axis=1)
    assert (m == 0).any()
    assert np.array_equal(out, brute.multiplicity_times_x(c.x, m))


def test_combine_renormalised_weights_identity_experts_recover_x():
    c = W.toy()
    slot, _, _ = oracle.slots(c.topk_idx, c.E, False, c.T * c.K)
    y = oracle.dispatch_bf16(c.x, slot, c.T * c.K)
    out = W.bf16_to_f32(oracle.combine(y, slot, c.topk_weights)).astype(np.float64)
    x = W.bf16_to_f32(c.x).astype(np.float64)
    # sum_k w = 1 up to fp32 rounding of the weights; one bf16 rounding at the end
    assert np.allclose(out, x, rtol=2.0 ** -8 + 1e-6, atol=1e-30)


def test_combine_empty_token_is_positive_zero():
    idx = np.array([[-1, -1], [0, 1]], np.int32)
    slot, _, _ = oracle.slots(idx, 2, False, 4)
    y = W.bf16_bits(np.full((4, 8), -1.5, np.float32))
    out = oracle.combine(y, slot, np.ones((2, 2), np.float32))
    assert (out[0] == 0x0000).all() and (out[1] == W.bf16_bits(np.float32([-3.0]))[0]).all()
