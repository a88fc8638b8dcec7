"""Seeded synthetic inputs for the MoE token dispatch/combine path.

This module makes inputs only.  It holds none of the dispatch/combine
arithmetic: it draws hidden rows ``x`` and stands in for the router that
produces ``topk_idx``/``topk_weights`` (token choice) or
``token_indices``/``weights`` (expert choice).  Both the HIP path and the CPU
oracle consume the arrays it returns, so it imports neither of them.

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream per workload,
draws in this fixed order):

1. ``x = standard_normal((T, H), float32)``, rounded to bf16 by torch's
   float32 -> bfloat16 cast (round to nearest even).
2. Router logits ``standard_normal((T, E))`` (token choice) or the expert
   scores ``z`` ``[T, E]`` then the token popularity ``b`` ``[T]`` (expert
   choice).
3. Token choice with skew: a per-expert bias from a Zipf law over a random
   rank ``r_e = permutation(E) + 1``: ``bias_e = c * log(r_e ** -s)``
   (the Zipf normaliser is a constant that does not change a top-K).
4. Optional -1 mask: exactly ``round(frac * T * K)`` flat slots drawn without
   replacement.

Top-K is taken in float64 over ``logits + bias``, in descending order, ties to
the lower expert index.  The weights are the softmax of the chosen K scores
(renormalised to sum 1 over the slots that survive the mask), stored as
float32.  Expert choice: ``token_indices[e]`` are the top-C tokens of
``score[:, e] = z[:, e] + 3 b`` (descending, ties to the lower token), and
``weights[e]`` the softmax over those C scores.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), via torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class TokenChoice:
    """A token-choice routing workload: x [T,H] bf16 bits, topk_idx [T,K]
    int32 (-1 = not dispatched), topk_weights [T,K] float32."""
    name: str
    T: int
    H: int
    E: int
    K: int
    x: np.ndarray
    topk_idx: np.ndarray
    topk_weights: np.ndarray
    layout: str = "contiguous"       # or "padded"
    quant: str = "bf16"              # or "fp8_e4m3_g128"
    cap: Optional[int] = None        # padded layout capacity per expert
    meta: dict = field(default_factory=dict)


@dataclass
class ExpertChoice:
    """An expert-choice routing workload: x [T,H] bf16 bits,
    token_indices [E,C] int32 (-1 = empty entry), weights [E,C] float32."""
    name: str
    T: int
    H: int
    E: int
    C: int
    x: np.ndarray
    token_indices: np.ndarray
    weights: np.ndarray
    meta: dict = field(default_factory=dict)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def router_topk(logits: np.ndarray, bias: Optional[np.ndarray], K: int):
    """Top-K experts per token of logits (+ bias) in float64, descending,
    ties to the lower expert index; weights = softmax of the chosen scores."""
    score = logits.astype(np.float64)
    if bias is not None:
        score = score + bias[None, :].astype(np.float64)
    order = np.argsort(-score, axis=1, kind="stable")[:, :K]
    chosen = np.take_along_axis(score, order, axis=1)
    return order.astype(np.int32), _softmax_rows(chosen)


def zipf_bias(rng: np.random.Generator, E: int, s: float, coef: float) -> np.ndarray:
    """bias_e = coef * log(Zipf_s pmf at a random rank r_e), up to a constant."""
    r = rng.permutation(E) + 1
    return coef * (-s) * np.log(r.astype(np.float64))


def make_token_choice(name: str, seed: int, T: int, H: int, E: int, K: int,
                      zipf_s: Optional[float] = None, zipf_coef: float = 1.0,
                      mask_frac: float = 0.0, **kw) -> TokenChoice:
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    bias = zipf_bias(rng, E, zipf_s, zipf_coef) if zipf_s is not None else None
    idx, w = router_topk(logits, bias, K)
    if mask_frac > 0.0:
        m = int(round(mask_frac * T * K))
        flat = rng.choice(T * K, size=m, replace=False)
        idx.reshape(-1)[flat] = -1
        w.reshape(-1)[flat] = 0.0
        tot = w.sum(axis=1, keepdims=True)
        w = np.divide(w, tot, out=np.zeros_like(w), where=tot > 0)
    return TokenChoice(name=name, T=T, H=H, E=E, K=K, x=x,
                       topk_idx=np.ascontiguousarray(idx, dtype=np.int32),
                       topk_weights=np.ascontiguousarray(w, dtype=np.float32), **kw)


def make_expert_choice(name: str, seed: int, T: int, H: int, E: int, C: int,
                       pop: float = 3.0) -> ExpertChoice:
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    z = rng.standard_normal((T, E))
    b = rng.standard_normal(T)
    score = z + pop * b[:, None]
    order = np.argsort(-score.T, axis=1, kind="stable")[:, :C]      # [E, C]
    chosen = np.take_along_axis(score.T, order, axis=1)
    w = _softmax_rows(chosen)
    return ExpertChoice(name=name, T=T, H=H, E=E, C=C, x=x,
                        token_indices=np.ascontiguousarray(order, dtype=np.int32),
                        weights=np.ascontiguousarray(w, dtype=np.float32))


# The five named workloads (DeepSeek-class MoE shapes: H=7168, E=256, top-8).
def toy(seed: int = 1) -> TokenChoice:
    """T=128, H=256, E=8, top-2, unbiased router; bf16 contiguous."""
    return make_token_choice("toy_T128_H256_E8_K2", seed, 128, 256, 8, 2)


def decode(seed: int = 2) -> TokenChoice:
    """T=128, H=7168, E=256, top-8; fp8 e4m3 (128-channel groups) into a
    padded [E, 128, H] buffer."""
    return make_token_choice("decode_T128_H7168_E256_K8_fp8_padded", seed, 128, 7168, 256, 8,
                             layout="padded", quant="fp8_e4m3_g128", cap=128)


def prefill(seed: int = 3) -> TokenChoice:
    """T=4096, H=7168, E=256, top-8, Zipf(1.2) bias with coefficient 2; bf16."""
    return make_token_choice("prefill_T4096_H7168_E256_K8", seed, 4096, 7168, 256, 8,
                             zipf_s=1.2, zipf_coef=2.0)


def expert_choice(seed: int = 4) -> ExpertChoice:
    """T=8192, H=4096, E=64, C=256, token popularity 3*N(0,1)."""
    return make_expert_choice("expert_choice_T8192_H4096_E64_C256", seed, 8192, 4096, 64, 256)


def large_padded(seed: int = 5) -> TokenChoice:
    """T=16384, H=7168, E=384, top-16, Zipf(1.1) bias, 15% of slots -1; bf16."""
    return make_token_choice("large_T16384_H7168_E384_K16_mask15", seed, 16384, 7168, 384, 16,
                             zipf_s=1.1, zipf_coef=1.0, mask_frac=0.15)


def as_token_choice(c: ExpertChoice) -> TokenChoice:
    """The token-centric form of an expert-choice workload, as a caller of a
    [T, K] API must build it ("[Feature Request] Support Expert-Choice
    Routing via Native Expert-Centric API", Current Limitation, item 2):
    topk_idx [T, K] lists the experts that picked each token in ascending
    order (ascending flat entry e*C + c), padded with -1 to K = the largest
    number of picks of any token; topk_weights carries each pick's weight
    and 0 on padding.  Host-side, outside any timed region."""
    T, E, C = c.T, c.E, c.C
    flat = c.token_indices.ravel()
    j = np.nonzero((flat >= 0) & (flat < T))[0]          # valid entries, ascending
    tok = flat[j].astype(np.int64)
    order = np.argsort(tok, kind="stable")               # by token, then ascending j
    j, tok = j[order], tok[order]
    m = np.bincount(tok, minlength=T)
    K = max(int(m.max()) if m.size else 0, 1)
    start = np.concatenate([[0], np.cumsum(m)[:-1]])
    k = np.arange(j.size) - start[tok]                   # rank inside the token
    idx = np.full((T, K), -1, np.int32)
    w = np.zeros((T, K), np.float32)
    idx[tok, k] = (j // C).astype(np.int32)
    w[tok, k] = c.weights.ravel()[j]
    return TokenChoice(name=f"{c.name}_as_token_choice_K{K}", T=T, H=c.H, E=E, K=K, x=c.x,
                       topk_idx=idx, topk_weights=w, layout="contiguous", quant="bf16",
                       meta={"from_expert_choice": c.name, "valid_entries": int(j.size)})


def expert_choice_tc() -> TokenChoice:
    """The expert-choice workload in token-centric form ([T, 64], mostly -1)."""
    return as_token_choice(expert_choice())


WORKLOADS = {"toy": toy, "decode": decode, "prefill": prefill,
             "expert_choice": expert_choice, "large_padded": large_padded,
             "expert_choice_tc": expert_choice_tc}


# Small random cases for parity sweeps: duplicates, -1 padding and invalid
# indices all occur.
def random_token_choice(seed: int, T: int, H: int, E: int, K: int, p_pad: float = 0.1,
                        p_invalid: float = 0.0, p_dup: float = 0.05) -> TokenChoice:
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    idx = rng.integers(0, E, size=(T, K), dtype=np.int64)
    if K > 1 and p_dup > 0:
        dup = rng.random((T, K)) < p_dup
        idx[:, 1:] = np.where(dup[:, 1:], idx[:, :-1], idx[:, 1:])
    u = rng.random((T, K))
    idx = np.where(u < p_pad, -1, idx)
    bad = (u >= p_pad) & (u < p_pad + p_invalid)
    badval = rng.choice(np.array([E, E + 7, -2, -100, 1 << 30], dtype=np.int64), size=(T, K))
    idx = np.where(bad, badval, idx)
    w = rng.random((T, K)).astype(np.float32)
    return TokenChoice(name=f"rand_T{T}_H{H}_E{E}_K{K}_s{seed}", T=T, H=H, E=E, K=K, x=x,
                       topk_idx=np.ascontiguousarray(idx, dtype=np.int32),
                       topk_weights=np.ascontiguousarray(w, dtype=np.float32))


def random_expert_choice(seed: int, T: int, H: int, E: int, C: int, p_empty: float = 0.1,
                         p_invalid: float = 0.0, hot: int = 0,
                         distinct: bool = False) -> ExpertChoice:
    """Uniform token picks (duplicates allowed, as with randint), optional
    -1 entries, invalid values, and `hot` tokens that every expert picks.
    With `distinct` (needs C <= T) no expert picks a token twice, as in
    top-C selection: each row is a random sample without replacement, and
    the hot tokens are distinct too."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    if distinct:
        assert C <= T
        h = min(hot, C)
        hot_set = rng.choice(T, size=h, replace=False)
        rest = np.setdiff1d(np.arange(T), hot_set)
        ti = np.empty((E, C), np.int64)
        for e in range(E):
            ti[e, :h] = hot_set
            ti[e, h:] = rng.choice(rest, size=C - h, replace=False)
            rng.shuffle(ti[e])
    else:
        ti = rng.integers(0, max(T, 1), size=(E, C), dtype=np.int64)
        if hot > 0 and T > 0:
            ti[:, :min(hot, C)] = rng.integers(0, T, size=min(hot, C))[None, :]
    u = rng.random((E, C))
    ti = np.where(u < p_empty, -1, ti)
    bad = (u >= p_empty) & (u < p_empty + p_invalid)
    ti = np.where(bad, T + 3, ti)
    if T == 0:
        ti[:] = -1
    w = rng.standard_normal((E, C)).astype(np.float32)
    return ExpertChoice(name=f"rand_ec_T{T}_H{H}_E{E}_C{C}_s{seed}", T=T, H=H, E=E, C=C, x=x,
                        token_indices=np.ascontiguousarray(ti, dtype=np.int32),
                        weights=np.ascontiguousarray(w, dtype=np.float32))
