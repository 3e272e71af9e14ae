"""Pins of the float64 causal-convolution oracle (oracle/conv_oracle.py) to facts
that do not come from the oracle itself: closed forms, a library convolution,
and the sequential, packing and replay invariants the pages list for the
compact convolution ("[CUDA] Add compact GatedDeltaNet operator", the embedded
VarlenCausalConv commit, Validation: sequential-prefix equivalence, all-ones
decode, adjacent requests, omitted output at zero capacity, capture counts,
capacity bounds)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import conv_oracle as CO


def _inputs(lengths, C=6, K=4, seed=0):
    rng = np.random.default_rng(seed)
    N = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return (rng.standard_normal((N, C)), rng.standard_normal((C, K)), rng.standard_normal(C), cu,
            rng.standard_normal((len(lengths), C, K - 1)))


def test_silu_closed_form():
    z = np.array([-3.0, -0.5, 0.0, 0.25, 4.0])
    assert np.allclose(CO.silu(z), z * (1.0 / (1.0 + np.exp(-z))), rtol=1e-15)
    assert CO.silu(0.0) == 0.0


def test_all_ones_decode():
    # x = 1, w = 1, s = 1: every output is SiLU(K + bias)
    C, K = 5, 4
    bias = np.linspace(-1, 1, C)
    out, fin, _ = CO.conv_forward(np.ones((3, C)), np.ones((C, K)), bias, [0, 1, 2, 3],
                                  np.ones((3, C, K - 1)))
    want = (K + bias) / (1 + np.exp(-(K + bias)))
    assert np.allclose(out, want[None, :], rtol=1e-15)
    assert np.array_equal(fin, np.ones((3, C, K - 1)))


def test_library_convolution():
    # per channel, the output before the activation is numpy's full convolution
    # of the carried-state-extended input with the reversed filter
    x, w, b, cu, s = _inputs([9], C=3, K=4, seed=1)
    out, _, _ = CO.conv_forward(x, w, b, cu, s, activation="none")
    for c in range(3):
        e = np.concatenate([s[0, c], x[:, c]])
        full = np.convolve(e, w[c, ::-1], mode="valid")            # sum_i w[i] e[j + i]
        assert np.allclose(out[:, c], full + b[c], rtol=1e-13, atol=1e-13)


def test_shift_and_identity_filters():
    x, _, _, cu, s = _inputs([7], C=2, K=4, seed=2)
    K = 4
    ident = np.zeros((2, K))
    ident[:, K - 1] = 1.0                                           # newest input
    out, _, _ = CO.conv_forward(x, ident, None, cu, s, activation="none")
    assert np.array_equal(out, x)
    oldest = np.zeros((2, K))
    oldest[:, 0] = 1.0                                              # input K - 1 steps back
    out, _, _ = CO.conv_forward(x, oldest, None, cu, s, activation="none")
    assert np.array_equal(out[K - 1:], x[:-(K - 1)])
    assert np.array_equal(out[:K - 1], s[0].T)


def test_sequential_prefix_equivalence():
    # the whole sequence equals token-by-token calls carrying the state
    x, w, b, cu, s = _inputs([11], seed=3)
    out, fin, _ = CO.conv_forward(x, w, b, cu, s)
    state = s
    for t in range(11):
        o1, state, _ = CO.conv_forward(x[t:t + 1], w, b, [0, 1], state)
        assert np.allclose(o1[0], out[t], rtol=1e-14, atol=1e-14)
    assert np.array_equal(state, fin)


def test_adjacent_requests_are_independent():
    x, w, b, cu, s = _inputs([5, 0, 3, 8], seed=4)
    out, fin, _ = CO.conv_forward(x, w, b, cu, s)
    for r in range(4):
        t0, t1 = cu[r], cu[r + 1]
        o1, f1, _ = CO.conv_forward(x[t0:t1], w, b, [0, t1 - t0], s[r:r + 1])
        assert np.array_equal(o1, out[t0:t1])
        assert np.array_equal(f1[0], fin[r])
    assert np.array_equal(fin[1], s[1])                             # empty request keeps its state


def test_short_request_final_state_mixes_state_and_inputs():
    x, w, b, cu, s = _inputs([2], C=3, K=4, seed=5)
    _, fin, _ = CO.conv_forward(x, w, b, cu, s)
    assert np.array_equal(fin[0], np.concatenate([s[0, :, 2:], x.T], axis=1))


def test_capture_and_replay_prefix():
    # replay of m captured values equals running the first m tokens
    cap = 4
    x, w, b, cu, s = _inputs([6, 3, 4], seed=6)
    _, _, capture = CO.conv_forward(x, w, b, cu, s, state_update_capacity=cap)
    for r in range(3):
        t0, L = cu[r], cu[r + 1] - cu[r]
        n = min(L, cap)
        assert np.array_equal(capture[r, :n], x[t0:t0 + n])
        for m in range(n + 1):
            _, fin_m, _ = CO.conv_forward(x[t0:t0 + m], w, b, [0, m], s[r:r + 1])
            rep = CO.conv_replay(s[r:r + 1], capture[r:r + 1], [m])
            assert np.array_equal(rep, fin_m)


def test_capture_count_and_zero_capacity():
    x, w, b, cu, s = _inputs([5, 5], seed=7)
    poison = np.full((2, 3, 6), -7.0)
    _, _, capture = CO.conv_forward(x, w, b, cu, s, state_update_capacity=3, capture_count=[1, 9],
                                    state_update_init=poison)
    assert np.array_equal(capture[0, 0], x[0]) and np.all(capture[0, 1:] == -7.0)
    assert np.array_equal(capture[1], x[5:8])                       # clamped to capacity
    _, _, none = CO.conv_forward(x, w, b, cu, s, state_update_capacity=0)
    assert none is None


def test_dense_layout():
    x, w, b, cu, s = _inputs([4, 4, 4], seed=8)
    a = CO.conv_forward(x, w, b, cu, s)
    d = CO.conv_forward(x, w, b, None, s, num_reqs=3)
    for u, v in zip(a[:2], d[:2]):
        assert np.array_equal(u, v)
    with pytest.raises(ValueError):
        CO.conv_forward(x, w, b, None, s, num_reqs=5)
