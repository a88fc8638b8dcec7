"""Deliberately naive numpy/Python brute force, independent of oracle/.

Each function restates a definition in the most direct way available (sorting
tuples, nearest-value search, per-element loops) so that a mistake in the C
oracle shows up as a disagreement.  Tiny inputs only.
"""
from __future__ import annotations

import numpy as np


def layout(topk_idx, E, R=1):
    T, K = topk_idx.shape
    valid = (topk_idx >= 0) & (topk_idx < E)
    counts = np.bincount(topk_idx[valid].astype(np.int64), minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    itr = np.zeros((T, R), np.uint8)
    per = E // R
    for t in range(T):
        for k in range(K):
            if valid[t, k]:
                itr[t, topk_idx[t, k] // per] = 1
    tpr = itr.sum(axis=0).astype(np.int32)
    ninv = int(((topk_idx != -1) & ~valid).sum())
    return dict(counts=counts, offsets=offsets, tokens_per_rank=tpr,
                is_token_in_rank=itr, num_invalid=ninv)


def slots(topk_idx, E, padded, cap_or_max_rows):
    """Sort the (e, t, k) tuples of valid entries; the position of a tuple in
    that order is its contiguous row; its position inside its expert is its
    rank r."""
    T, K = topk_idx.shape
    tuples = sorted((int(topk_idx[t, k]), t, k) for t in range(T) for k in range(K)
                    if 0 <= topk_idx[t, k] < E)
    slot = np.full((T, K), -1, np.int32)
    first = {}
    dropped = 0
    for pos, (e, t, k) in enumerate(tuples):
        first.setdefault(e, pos)
        r = pos - first[e]
        if padded:
            s = e * cap_or_max_rows + r if r < cap_or_max_rows else -1
        else:
            s = pos if pos < cap_or_max_rows else -1
        if s < 0:
            dropped += 1
        slot[t, k] = s
    return slot, dropped


# ------------------------------------------------------------- e4m3 / bf16
def e4m3_table():
    """Value of every E4M3 code from the bit-field definition: bias 7,
    3 mantissa bits, exponent field 0 = subnormal, S.1111.111 = NaN."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s, ef, m = c >> 7, (c >> 3) & 15, c & 7
        if ef == 15 and m == 7:
            v = np.nan
        elif ef == 0:
            v = m / 8.0 * 2.0 ** (1 - 7)
        else:
            v = (1 + m / 8.0) * 2.0 ** (ef - 7)
        vals[c] = -v if s else v
    return vals


def e4m3_nearest(v):
    """Nearest finite E4M3 code to each fp32 value (searching all codes of
    the value's sign), ties to the even code; magnitudes above 448 saturate
    to 448.  Vectorised brute-force search."""
    v = np.asarray(v, np.float32).astype(np.float64)
    tab = e4m3_table()
    pos_codes = np.array([c for c in range(128) if not np.isnan(tab[c])])   # 0x00..0x7E
    pos_vals = tab[pos_codes]
    a = np.minimum(np.abs(v), 448.0 * 2)  # beyond 448 every search returns 448
    d = np.abs(a[:, None] - pos_vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer the even code
    even = (pos_codes % 2 == 0)[None, :]
    pick_even = cand & even
    has_even = pick_even.any(axis=1)
    choose = np.where(has_even[:, None], pick_even, cand)
    code = pos_codes[np.argmax(choose, axis=1)]
    sign = np.signbit(v)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def bf16_nearest_f64(v):
    """Nearest bf16 to a float64 value by listing the two bf16 neighbours
    (truncation and next-up in fp32 bit space), ties to even."""
    out = np.empty(len(v), np.uint16)
    for i, x in enumerate(np.asarray(v, np.float64)):
        if x == 0:
            out[i] = 0x8000 if np.signbit(x) else 0
            continue
        a = abs(x)
        # bf16 candidates around a: take the fp32 just below/above, truncate
        lo_bits = np.array([a], np.float32).view(np.uint32)[0] & 0xFFFF0000
        lo = float(np.array([lo_bits], np.uint32).view(np.float32)[0])
        if lo > a:
            lo_bits -= 0x10000
            lo = float(np.array([lo_bits], np.uint32).view(np.float32)[0])
        hi_bits = lo_bits + 0x10000
        hi = float(np.array([hi_bits], np.uint32).view(np.float32)[0])
        if a - lo < hi - a:
            b = lo_bits
        elif hi - a < a - lo:
            b = hi_bits
        else:
            b = lo_bits if ((lo_bits >> 16) & 1) == 0 else hi_bits
        b = int(b) >> 16
        out[i] = b | (0x8000 if x < 0 else 0)
    return out


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp8_quant_token(xrow_bits):
    """Per-128-channel e4m3 quantisation of one bf16 row, written with
    numpy float32 arithmetic and the brute-force encoder."""
    x = bf16_to_f64(xrow_bits).astype(np.float32)
    H = x.size
    q = np.empty(H, np.uint8)
    s = np.empty(H // 128, np.float32)
    for g in range(H // 128):
        blk = x[128 * g:128 * (g + 1)]
        a = np.float32(np.abs(blk).max())
        if a == 0:
            s[g] = 0
            q[128 * g:128 * (g + 1)] = 0
            continue
        sg = np.float32(a / np.float32(448.0))
        s[g] = sg
        q[128 * g:128 * (g + 1)] = e4m3_nearest((blk / sg).astype(np.float32))
    return q, s


def combine_f64(y_bits, slot, w):
    """Per-element loops, fp64 sums, rounded to bf16 by bf16_nearest_f64."""
    T, K = slot.shape
    H = y_bits.shape[1]
    acc = np.zeros((T, H), np.float64)
    yf = bf16_to_f64(y_bits)
    for t in range(T):
        for k in range(K):
            s = slot[t, k]
            if s >= 0:
                acc[t] += (1.0 if w is None else float(w[t, k])) * yf[s]
    return bf16_nearest_f64(acc.ravel()).reshape(T, H)


def ec_invert(token_indices, T):
    flat = token_indices.reshape(-1)
    valid = (flat >= 0) & (flat < T)
    j = np.nonzero(valid)[0]
    order = np.argsort(flat[j], kind="stable")      # CSR transpose by stable sort
    ent = j[order].astype(np.int32)
    off = np.concatenate([[0], np.cumsum(np.bincount(flat[j], minlength=T))]).astype(np.int32)
    return off, ent


def multiplicity_times_x(x_bits, m):
    """bf16(m_t * x_t) per row, where a zero result is +0: the sum starts
    from +0, and +0 + (-0) = +0, so neither a token nobody received nor a
    sum of -0 terms gives -0.  m_t * x_t is exact in fp32 for m_t <= 2^16;
    numpy forms it and torch's cast rounds it to bf16."""
    import torch
    xf = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    prod = (xf * np.asarray(m, np.float32)[:, None]).astype(np.float32)
    prod = np.where(prod == 0, np.float32(0.0), prod)
    return torch.from_numpy(np.ascontiguousarray(prod)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _nearest_code(v, codes, vals, maxv, sign_bit):
    """Nearest code to each value among (codes, vals) of non-negative
    magnitudes, ties to the even code, magnitudes above maxv saturating."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 2.0 * maxv)
    d = np.abs(a[:, None] - vals[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = (codes % 2 == 0)[None, :]
    pick_even = cand & even
    choose = np.where(pick_even.any(axis=1)[:, None], pick_even, cand)
    code = codes[np.argmax(choose, axis=1)]
    return (code | np.where(np.signbit(v), sign_bit, 0)).astype(np.uint8)


def e5m2_table():
    """Value of every non-negative finite E5M2 code 0x00..0x7B, listed from
    the bit fields: exponent field f (bias 15), 2 fraction bits."""
    codes = np.arange(0x7C)
    vals = np.array([(c & 3) * 2.0 ** -16 if (c >> 2) == 0 else (1 + (c & 3) / 4) * 2.0 ** ((c >> 2) - 15)
                     for c in codes])
    return codes, vals


def e5m2_nearest(v):
    codes, vals = e5m2_table()
    return _nearest_code(v, codes, vals, 57344.0, 0x80)


def e2m1_nearest(v):
    codes = np.arange(8)
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    return _nearest_code(v, codes, vals, 6.0, 0x8)


def int8_token_quant(xrow_bits):
    """Per-token int8: numpy float32 division and np.rint (half to even)."""
    x = bf16_to_f64(xrow_bits).astype(np.float32)
    a = np.float32(np.abs(x).max())
    if a == 0:
        return np.zeros(x.size, np.uint8), np.float32(0)
    s = np.float32(a / np.float32(127.0))
    q = np.clip(np.rint((x / s).astype(np.float32)), -127, 127).astype(np.int8)
    return q.view(np.uint8), s


def mx_quant_row(xrow_bits, fmt):
    """MX quantisation of one row with numpy: block exponent from np.frexp,
    exact scaling by np.ldexp, elements by brute-force nearest-code search."""
    emax = {"mxfp8_e4m3": 8, "mxfp8_e5m2": 15, "mxfp4_e2m1": 2}[fmt]
    near = {"mxfp8_e4m3": e4m3_nearest, "mxfp8_e5m2": e5m2_nearest, "mxfp4_e2m1": e2m1_nearest}[fmt]
    x = bf16_to_f64(xrow_bits)
    H = x.size
    codes = np.zeros(H, np.uint8)
    ecode = np.zeros(H // 32, np.uint8)
    for b in range(H // 32):
        blk = x[32 * b:32 * (b + 1)]
        a = np.abs(blk).max()
        E = -127
        if a > 0:
            E = int(np.clip(np.frexp(a)[1] - 1 - emax, -127, 127))
        ecode[b] = E + 127
        scaled = np.ldexp(blk, -E)
        if fmt == "mxfp8_e4m3":
            # e4m3_nearest takes fp32; scaled values below fp32's range only
            # occur far below the smallest subnormal code, where they give 0
            codes[32 * b:32 * (b + 1)] = near(scaled.astype(np.float32))
        else:
            codes[32 * b:32 * (b + 1)] = near(scaled)
    if fmt == "mxfp4_e2m1":
        codes = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return codes, ecode


# ------------------------------------------------------------- one rank's share
def rank_pack(topk_idx, w, E, R, max_rows):
    """Sort the distinct (rank, token) pairs of valid entries; the position
    of a pair in that order is its send row.  Each row carries the token's
    entries with the experts of that rank as local ids, -1 elsewhere."""
    T, K = topk_idx.shape
    per = E // R
    pairs = sorted({(int(topk_idx[t, k]) // per, t) for t in range(T) for k in range(K)
                    if 0 <= topk_idx[t, k] < E})
    off = np.array([sum(1 for r_, _ in pairs if r_ < r) for r in range(R + 1)], np.int32)
    pos = np.full((T, R), -1, np.int32)
    rows = []
    for p, (r, t) in enumerate(pairs):
        if p >= max_rows:
            continue
        pos[t, r] = p
        ids = [int(topk_idx[t, k]) - r * per
               if 0 <= topk_idx[t, k] < E and topk_idx[t, k] // per == r else -1
               for k in range(K)]
        ws = [(1.0 if w is None else float(w[t, k])) if ids[k] >= 0 else 0.0 for k in range(K)]
        rows.append((t, ids, ws))
    return dict(rank_offsets=off, pack_pos=pos, rows=rows,
                num_dropped=max(0, len(pairs) - max_rows))


def combine_partial_f64(y_bits, slot, w):
    """Per-element loops, fp64 sums, rounded once to fp32."""
    S, K = slot.shape
    yf = bf16_to_f64(y_bits)
    acc = np.zeros((S, y_bits.shape[1]), np.float64)
    for p in range(S):
        for k in range(K):
            if slot[p, k] >= 0:
                acc[p] += (1.0 if w is None else float(w[p, k])) * yf[slot[p, k]]
    return acc.astype(np.float32)


def combine_ranks_f64(partial, pack_pos):
    """Per token, the partial rows of its ranks summed in rank order (fp64),
    rounded once to bf16."""
    T, R = pack_pos.shape
    acc = np.zeros((T, partial.shape[1]), np.float64)
    for t in range(T):
        for r in range(R):
            p = pack_pos[t, r]
            if 0 <= p < partial.shape[0]:
                acc[t] += partial[p].astype(np.float64)
    return bf16_nearest_f64(acc.ravel()).reshape(acc.shape)
