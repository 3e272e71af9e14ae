"""Pins of the pooled fixed-state oracle (oracle/pool_oracle.py) to facts that do
not come from its own code: the request-indexed oracle in the special cases the
pooled form reduces to, slot permutations, untouched slots, and the
double-buffered speculative step of "Replay compact fixed state for hybrid
decoding" (Key Changes: per-request ownership, double-buffered publication,
compact prefix replay), whose committed state after publication must equal a
plain forward over the accepted prefix."""
from __future__ import annotations

import numpy as np

from gdn_workloads import make_inputs
from gdn_workloads.conv import make_conv_inputs
from oracle import conv_oracle as CO
from oracle import gdn_oracle as GO
from oracle import pool_oracle as PO


def _gdn(lengths, seed, capacity=0):
    return make_inputs(lengths, 1, 2, 8, 6, "f32", seed=seed, capacity=capacity)


def _fwd_args(inp):
    return [inp[n] for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")]


def test_identity_slots_reduce_to_request_indexed():
    inp = _gdn([3, 1, 4], seed=1)
    o, pool, _ = PO.gdn_forward_pooled(*_fwd_args(inp), inp["initial_state"], None, None)
    o_ref, s_ref, _ = GO.gdn_forward(*_fwd_args(inp), inp["initial_state"])
    assert np.array_equal(o, o_ref) and np.array_equal(pool, s_ref)


def test_slot_permutation_and_untouched_slots():
    inp = _gdn([2, 5, 1], seed=2)
    rng = np.random.default_rng(0)
    P = 7
    pool = rng.standard_normal((P,) + inp["initial_state"].shape[1:])
    rd, wr = np.array([4, 0, 6]), np.array([1, 3, 5])
    o, out_pool, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool, rd, wr)
    o_ref, s_ref, _ = GO.gdn_forward(*_fwd_args(inp), pool[rd])
    assert np.array_equal(o, o_ref)
    assert np.array_equal(out_pool[wr], s_ref)
    untouched = [s for s in range(P) if s not in wr]
    assert np.array_equal(out_pool[untouched], pool[untouched])


def test_missing_slot_reads_zero_and_writes_nothing():
    inp = _gdn([3, 2], seed=3)
    pool = np.ones((3,) + inp["initial_state"].shape[1:])
    o, out_pool, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool, [-1, 2], [0, -1])
    S0 = np.stack([np.zeros(pool.shape[1:]), pool[2]])
    o_ref, s_ref, _ = GO.gdn_forward(*_fwd_args(inp), S0)
    assert np.array_equal(o, o_ref)
    assert np.array_equal(out_pool[0], s_ref[0])
    assert np.array_equal(out_pool[1:], pool[1:])


def test_publish_swaps_and_twice_is_identity():
    c, i = np.array([0, 2, 4]), np.array([1, 3, 5])
    c1, i1 = PO.publish(c, i)
    assert np.array_equal(c1, i) and np.array_equal(i1, c)
    c2, i2 = PO.publish(c1, i1)
    assert np.array_equal(c2, c) and np.array_equal(i2, i)


def test_double_buffered_step_equals_prefix_forward():
    # verify 4 draft tokens per request against the committed slots, replay the
    # accepted prefix into the inactive slots, publish: the committed state is then
    # the state after exactly the accepted tokens
    T, R, cap = 4, 3, 4
    inp = _gdn([T] * R, seed=4, capacity=cap)
    rng = np.random.default_rng(5)
    P = 2 * R
    pool = np.zeros((P,) + inp["initial_state"].shape[1:])
    committed, inactive = np.array([1, 2, 5]), np.array([0, 3, 4])
    pool[committed] = inp["initial_state"]
    accepted = np.array([0, 2, 4])
    _, _, capsule = PO.gdn_forward_pooled(*_fwd_args(inp), pool, committed, [-1] * R,
                                          state_update_capacity=cap)
    pool = PO.gdn_replay_pooled(pool, capsule, accepted, committed, inactive, 1, 2, 8, 6)
    committed, inactive = PO.publish(committed, inactive)
    for r in range(R):
        m, t0 = int(accepted[r]), int(inp["cu_seqlens"][r])
        sl = slice(t0, t0 + m)
        _, s_ref, _ = GO.gdn_forward(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["a"][sl], inp["b"][sl],
                                     inp["A_log"], inp["dt_bias"], [0, m], inp["initial_state"][r:r + 1])
        np.testing.assert_allclose(pool[committed[r]], s_ref[0], rtol=1e-12, atol=1e-13)
        # the previously committed slot is untouched until it is reused
        assert np.array_equal(pool[inactive[r]], inp["initial_state"][r])


def test_conv_double_buffered_step_equals_prefix_forward():
    T, R, cap = 4, 3, 4
    inp = make_conv_inputs([T] * R, 8, 4, "f32", seed=6, capacity=cap)
    P = 2 * R
    pool = np.zeros((P, 8, 3))
    committed, inactive = np.array([3, 0, 5]), np.array([1, 2, 4])
    pool[committed] = inp["initial_state"]
    accepted = np.array([1, 4, 0])
    _, _, capture = PO.conv_forward_pooled(inp["x"], inp["weight"], inp["bias"], inp["cu_seqlens"],
                                           pool, committed, [-1] * R, state_update_capacity=cap)
    pool = PO.conv_replay_pooled(pool, capture, accepted, committed, inactive)
    committed, _ = PO.publish(committed, inactive)
    for r in range(R):
        m, t0 = int(accepted[r]), int(inp["cu_seqlens"][r])
        _, fin, _ = CO.conv_forward(inp["x"][t0:t0 + m], inp["weight"], inp["bias"], [0, m],
                                    inp["initial_state"][r:r + 1])
        assert np.array_equal(pool[committed[r]], fin[0])
