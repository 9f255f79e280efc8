"""The parity helpers themselves (CPU only): the argmax validity check must
reject every wrong answer a pooled output can carry, near-tie windows
included, and accept every right one.  Values come from the fp64 oracle on a
tiny softmax + two-pool problem (page "Kimi-K2.6__l2_p6"), and the wrong
answers are planted into copies of the oracle's own outputs."""
import numpy as np
import pytest

import cnf_inputs
import oracle
from parity import check_argmax, oracle_pre_pool


def _problem():
    wl = cnf_inputs.workload("conv3d_softmax_pool_n128", N=1, in_dims=(8, 8, 8))
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    out, idx = oracle.forward(wl, x, **p)
    pre = oracle_pre_pool(wl, x, p)
    return out, idx, pre


def test_oracle_answer_passes():
    out, idx, pre = _problem()
    assert check_argmax(idx, out, idx, pre, 4, "oracle") >= 0


def test_wrong_index_in_clear_window_fails():
    out, idx, pre = _problem()
    bad = idx.copy()
    # another voxel of the same window (flat d*H*W + h*W + w on the 6x6x6 conv grid)
    bad[0, 0, 0, 0, 0] = idx[0, 0, 0, 0, 0] ^ 1
    with pytest.raises(AssertionError):
        check_argmax(bad, out, idx, pre, 4, "planted")


def test_index_outside_window_fails():
    out, idx, pre = _problem()
    bad = idx.copy()
    bad[0, 1, 0, 0, 0] = 5 * 36 + 5 * 6 + 5 + 1000   # past the grid
    with pytest.raises(AssertionError):
        check_argmax(bad, out, idx, pre, 4, "planted")


def test_near_tie_window_index_below_max_fails():
    # make one window a near-tie in a copy of the oracle's pre-pool values; an
    # index naming a voxel far below the maximum must still be rejected
    out, idx, pre = _problem()
    pre = pre.copy()
    i0 = int(idx[0, 2, 0, 0, 0])
    d, h, w = i0 // 36, (i0 // 6) % 6, i0 % 6
    other = [(a, b, c) for a in range(4) for b in range(4) for c in range(4) if (a, b, c) != (d, h, w)]
    a, b, c = other[0]
    pre[0, 2, a, b, c] = pre[0, 2, d, h, w] - 1e-6          # near-tie partner: valid
    a2, b2, c2 = other[1]
    pre[0, 2, a2, b2, c2] = pre[0, 2, d, h, w] - 0.5        # clearly below the max
    tie_ok = idx.copy()
    tie_ok[0, 2, 0, 0, 0] = a * 36 + b * 6 + c
    vals = out.copy()
    vals[0, 2, 0, 0, 0] = pre[0, 2, a, b, c]
    check_argmax(tie_ok, vals, idx, pre, 4, "tie partner")     # accepted
    bad = idx.copy()
    bad[0, 2, 0, 0, 0] = a2 * 36 + b2 * 6 + c2
    with pytest.raises(AssertionError):
        check_argmax(bad, out, idx, pre, 4, "below max")


def test_pooled_value_must_match_own_index():
    out, idx, pre = _problem()
    vals = out.copy()
    vals[0, 3, 0, 0, 0] += 1e-2
    with pytest.raises(AssertionError):
        check_argmax(idx, vals, idx, pre, 4, "value")
    assert np.isfinite(vals).all()
