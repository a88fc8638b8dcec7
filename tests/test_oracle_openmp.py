"""The -fopenmp build of the oracle (the all-host-cores CPU baseline) gives
the same bytes as the plain single-threaded build, op by op."""
import numpy as np

import oracle
from combine_get_dispatch_04_amd import workloads as W


def _token_choice_ops(c, rows):
    s, src, nd = oracle.slots(c.topk_idx, c.E, False, rows)
    y = oracle.dispatch_bf16(c.x, s, rows)
    out = [oracle.layout(c.topk_idx, c.E, 4)["offsets"], s, src, y,
           *oracle.dispatch_fp8(c.x, s, rows),
           *oracle.dispatch_token_quant(c.x, s, rows, "int8_token"),
           *oracle.dispatch_token_quant(c.x, s, rows, "fp8_e4m3_token"),
           *oracle.dispatch_mx(c.x, s, rows, "mxfp8_e5m2"),
           *oracle.dispatch_mx(c.x, s, rows, "mxfp4_e2m1"),
           oracle.combine(y, s, c.topk_weights), oracle.combine(y, s, None)]
    return out


def _expert_choice_ops(c):
    recv, ninv = oracle.ec_dispatch(c.x, c.token_indices)
    off, ent = oracle.ec_invert(c.token_indices, c.T)
    return [recv, np.array([ninv]), off, ent,
            oracle.ec_combine(recv, c.weights, c.token_indices, c.T)]


def _same(a_list, b_list):
    assert len(a_list) == len(b_list)
    for i, (a, b) in enumerate(zip(a_list, b_list)):
        assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8)), i


def test_openmp_build_equals_plain_build():
    tc = W.random_token_choice(11, 1500, 1024, 48, 6, p_pad=0.1, p_invalid=0.02, p_dup=0.1)
    tc.topk_idx[7, 2] = 10 ** 6          # an invalid entry
    ec = W.random_expert_choice(12, 900, 256, 24, 64, p_empty=0.1, hot=8)
    ec.token_indices[3, 5] = -7          # an invalid entry
    plain = _token_choice_ops(tc, tc.T * tc.K - 100), _expert_choice_ops(ec)
    with oracle.all_cores() as threads:
        assert threads >= 1
        par = _token_choice_ops(tc, tc.T * tc.K - 100), _expert_choice_ops(ec)
    _same(plain[0], par[0])
    _same(plain[1], par[1])
    # the plain build is back in force after the block
    assert oracle.lib().oracle_max_threads() == 1
