"""Pins of the float64 oracle against closed forms, invariants and brute force.

Each check reads the oracle's functions at call time, so the planted-mistake
tests in test_oracle_mutations.py can swap one in and see a check fail.
"""
from __future__ import annotations

import json
import math
import os
import warnings

import numpy as np
import pytest
from scipy.special import expit

import brute_force as bf
from gdn_workloads import cu_from_lengths, make_inputs
from oracle import gdn_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-11


def _rel(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-300))


def _tiny(lengths, Hk=1, Hv=1, Dk=6, Dv=5, seed=11, initial="normal", capacity=0):
    return make_inputs(lengths, Hk, Hv, Dk, Dv, "f32", seed, initial=initial, capacity=capacity)


def _forward(inp, **kw):
    return O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                         inp["dt_bias"], inp["cu_seqlens"], inp["initial_state"], **kw)


# ---------------------------------------------------------------- P-1 gates
def check_gate_closed_form():
    rng = np.random.default_rng(0)
    Hv = 5
    a = rng.standard_normal((40, Hv)) * 3.0
    b = rng.standard_normal((40, Hv)) * 3.0
    A_log = np.log(rng.uniform(1.0, 16.0, Hv))
    dt_bias = rng.uniform(-1.0, 1.0, Hv)
    alpha, beta = O.gates(a, b, A_log, dt_bias)
    alpha_ref, beta_ref = bf.closed_form_gates(a, b, A_log, dt_bias)
    assert _rel(alpha, alpha_ref) < 1e-12
    assert np.allclose(beta, beta_ref, rtol=1e-14, atol=0)
    assert np.allclose(beta, expit(b), rtol=1e-14, atol=0)       # library sigmoid
    assert np.all((alpha > 0) & (alpha <= 1))
    # special values: x = 0 gives alpha = 2^-A, b = 0 gives beta = 1/2
    A_log1 = np.array([math.log(3.0)])
    al0, be0 = O.gates(np.array([[0.25]]), np.array([[0.0]]), A_log1, np.array([-0.25]))
    assert abs(al0[0, 0] - 2.0 ** -3.0) < 1e-15 and be0[0, 0] == 0.5
    # large x: softplus(x) -> x, so log alpha -> -A x
    la = O.log_decay(np.array([[60.0]]), np.array([0.0]), np.array([0.0]))
    assert abs(la[0, 0] + 60.0) < 1e-12


def test_gate_closed_form():
    check_gate_closed_form()


def test_softplus_against_direct_formula():
    x = np.linspace(-30, 30, 601)
    assert np.allclose(O.softplus(x), np.log1p(np.exp(x)), rtol=1e-13, atol=1e-300)
    assert O.softplus(np.array([800.0]))[0] == 800.0        # no overflow
    assert O.softplus(np.array([0.0]))[0] == math.log(2.0)


# ------------------------------------------------------- P-2 normalisation
def check_normalisation():
    inp = _tiny([7], Hk=2, Hv=4, Dk=8, Dv=3)
    k = inp["k"].astype(np.float64)
    kh = O.l2normalize(k)
    nk = np.sum(k * k, axis=-1)
    assert np.allclose(np.sum(kh * kh, axis=-1), nk / (nk + O.L2NORM_EPS), rtol=1e-14)
    # one token from a zero state: o = beta v (k^ . q^) with q^ carrying Dk^-1/2 (P-6)
    one = _tiny([1], Hk=1, Hv=1, Dk=8, Dv=3, initial="zero")
    out, fin, _ = _forward(one)
    q = one["q"][0, 0].astype(np.float64)
    kk = one["k"][0, 0].astype(np.float64)
    _, beta = bf.closed_form_gates(one["a"], one["b"], one["A_log"], one["dt_bias"])
    expect = beta[0, 0] * one["v"][0, 0] * float(bf.unit(kk) @ bf.unit(q)) / math.sqrt(8)
    assert _rel(out[0, 0], expect) < TIGHT
    assert _rel(fin[0, 0], beta[0, 0] * np.outer(one["v"][0, 0], bf.unit(kk))) < TIGHT


def test_normalisation_and_scale():
    check_normalisation()


def test_explicit_scale_is_used():
    one = _tiny([3], Dk=8, Dv=3)
    o1, _, _ = _forward(one, scale=0.5)
    o2, _, _ = _forward(one, scale=0.25)
    # the output is linear in the query scale; the state does not depend on it
    assert _rel(o1, 2.0 * o2) < TIGHT


# ------------------------------------------------- P-3 / P-4 frozen, decay
def check_frozen_state():
    rng = np.random.default_rng(1)
    T, H, Dk, Dv = 9, 3, 6, 4
    qh = rng.standard_normal((T, H, Dk))
    kh = O.l2normalize(rng.standard_normal((T, H, Dk)))
    v = rng.standard_normal((T, H, Dv))
    S0 = rng.standard_normal((H, Dv, Dk))
    o, S, u = O.recurrence(qh, kh, v, np.ones((T, H)), np.zeros((T, H)), S0)
    assert np.array_equal(S, S0)
    assert np.allclose(o, np.einsum("hvk,thk->thv", S0, qh), rtol=1e-13, atol=1e-13)
    assert np.all(u == 0)
    # the same through the raw gate inputs: A_log = -inf gives alpha = 1,
    # b = -inf gives beta = 0
    inp = _tiny([5, 4], Hk=1, Hv=2, Dk=6, Dv=4)
    inp["A_log"] = np.full(2, -np.inf)
    inp["b"] = np.full_like(inp["b"], -np.inf)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        out, fin, _ = _forward(inp)
    assert np.array_equal(fin, inp["initial_state"].astype(np.float64))
    for r, (t0, t1) in enumerate(zip(inp["cu_seqlens"][:-1], inp["cu_seqlens"][1:])):
        for t in range(t0, t1):
            qn = O.l2normalize(inp["q"][t, 0].astype(np.float64)) / math.sqrt(6)
            assert _rel(out[t], inp["initial_state"][r] @ qn) < TIGHT


def test_frozen_state():
    check_frozen_state()


def check_decay_only():
    inp = _tiny([6], Hk=1, Hv=2, Dk=5, Dv=4)
    inp["b"] = np.full_like(inp["b"], -np.inf)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        out, fin, _ = _forward(inp)
    alpha, _ = bf.closed_form_gates(inp["a"], np.zeros_like(inp["b"]), inp["A_log"], inp["dt_bias"])
    gamma = np.prod(alpha, axis=0)                                # [Hv]
    assert _rel(fin[0], gamma[:, None, None] * inp["initial_state"][0]) < TIGHT


def test_decay_only():
    check_decay_only()


# ------------------------------------------------------- P-5 exact write
def check_exact_write():
    rng = np.random.default_rng(2)
    Dk, Dv, n = 8, 5, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:, :n].T                                            # orthonormal rows
    v = rng.standard_normal((n, 1, Dv))
    S0 = rng.standard_normal((1, Dv, Dk))
    qh = rng.standard_normal((n, 1, Dk))
    o, S, _ = O.recurrence(qh, keys[:, None, :], v, np.ones((n, 1)), np.ones((n, 1)), S0)
    for i in range(n):
        assert np.allclose(S[0] @ keys[i], v[i, 0], rtol=0, atol=1e-12)
    for x in Qm[:, n:].T:                                         # orthogonal complement
        assert np.allclose(S[0] @ x, S0[0] @ x, rtol=0, atol=1e-12)


def test_exact_write():
    check_exact_write()


# ------------------------------------------------ P-7 brute force (tiny)
def _per_head_brute(inp, form):
    """Run a brute-force form on every (sequence, value head); packed outputs."""
    q, k, v = (inp[n].astype(np.float64) for n in ("q", "k", "v"))
    Hk, Hv, Dk, Dv = inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"]
    alpha, beta = bf.closed_form_gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    R = len(cu) - 1
    out = np.zeros((q.shape[0], Hv, Dv))
    fin = np.zeros((R, Hv, Dv, Dk))
    G = Hv // Hk
    for r in range(R):
        t0, t1 = cu[r], cu[r + 1]
        for h in range(Hv):
            S0 = (np.zeros((Dv, Dk)) if inp["initial_state"] is None
                  else inp["initial_state"][r, h].astype(np.float64))
            if t1 == t0:
                fin[r, h] = S0
                continue
            res = form(q[t0:t1, h // G], k[t0:t1, h // G], v[t0:t1, h], alpha[t0:t1, h],
                       beta[t0:t1, h], S0, 1.0 / math.sqrt(Dk))
            out[t0:t1, h] = res[0]
            fin[r, h] = res[1][-1] if res[1].ndim == 3 else res[1]
    return out, fin


def check_transition_form():
    inp = _tiny([5, 0, 9, 1], Hk=2, Hv=4, Dk=6, Dv=5, seed=21)
    out, fin, _ = _forward(inp)
    ob, fb = _per_head_brute(inp, bf.transition_form)
    assert _rel(out, ob) < TIGHT and _rel(fin, fb) < TIGHT


def test_transition_form():
    check_transition_form()


def check_materialised_form():
    inp = _tiny([12, 3], Hk=1, Hv=3, Dk=7, Dv=4, seed=22)
    out, fin, _ = _forward(inp)
    ob, fb = _per_head_brute(inp, bf.materialised_form)
    assert _rel(out, ob) < 1e-10 and _rel(fin, fb) < 1e-10


def test_materialised_form():
    check_materialised_form()


# ---------------------------------------------- P-8 chunked == recurrent
def check_chunked_equals_recurrent(chunks=(1, 7, 16, 64, 200)):
    inp = _tiny([150, 1, 64, 65, 0, 37], Hk=2, Hv=4, Dk=8, Dv=6, seed=23)
    out, fin, _ = _forward(inp)
    for C in chunks:
        oc, fc = O.chunked_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                   inp["A_log"], inp["dt_bias"], inp["cu_seqlens"],
                                   inp["initial_state"], chunk=C)
        assert _rel(oc, out) < 1e-10, C
        assert _rel(fc, fin) < 1e-10, C


def test_chunked_equals_recurrent():
    check_chunked_equals_recurrent()


def test_chunked_with_strong_decay():
    """Decays down to e^-100 per token stay finite in the log-space chunk form."""
    inp = _tiny([130], Hk=1, Hv=2, Dk=8, Dv=4, seed=24)
    inp["A_log"] = np.log(np.array([16.0, 16.0], np.float32))
    inp["a"] = inp["a"] + np.float32(5.0)
    out, fin, _ = _forward(inp)
    oc, fc = O.chunked_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                               inp["dt_bias"], inp["cu_seqlens"], inp["initial_state"], chunk=64)
    assert np.all(np.isfinite(oc)) and _rel(oc, out) < 1e-10 and _rel(fc, fin) < 1e-10


# ------------------------------------------- capsule layout and P-9 replay
def check_capsule_layout():
    Hk, Hv, Dk, Dv, cap = 2, 4, 6, 5, 3
    inp = _tiny([4, 2, 0, 5], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, seed=25, capacity=cap)
    R = 4
    W = O.capsule_width(Hk, Hv, Dk, Dv)
    assert W == Hv + Hk * Dk + Hv * Dv
    poison = np.full((R, cap, W), 7.5)
    capture = np.array([3, 1, 2, 0])
    _, _, capsule = _forward(inp, state_update_capacity=cap, capture_count=capture,
                             state_update_init=poison)
    alpha, _ = bf.closed_form_gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    q, k, v = (inp[n].astype(np.float64) for n in ("q", "k", "v"))
    cu = inp["cu_seqlens"]
    G = Hv // Hk
    for r in range(R):
        t0, t1 = cu[r], cu[r + 1]
        n = min(t1 - t0, capture[r])
        for j in range(cap):
            row = capsule[r, j]
            if j >= n:
                assert np.all(row == 7.5)               # rows past n_r untouched
                continue
            t = t0 + j
            assert np.allclose(row[:Hv], alpha[t], rtol=1e-13)
            for g in range(Hk):
                assert np.allclose(row[Hv + g * Dk: Hv + (g + 1) * Dk], bf.unit(k[t, g]), rtol=1e-13)
            for h in range(Hv):
                S0 = inp["initial_state"][r, h].astype(np.float64)
                _, _, deltas = bf.transition_form(q[t0:t1, h // G], k[t0:t1, h // G], v[t0:t1, h],
                                                  alpha[t0:t1, h],
                                                  bf.closed_form_gates(inp["a"], inp["b"], inp["A_log"],
                                                                       inp["dt_bias"])[1][t0:t1, h],
                                                  S0, 1.0 / math.sqrt(Dk))
                d0 = Hv + Hk * Dk + h * Dv
                assert _rel(row[d0:d0 + Dv], deltas[j]) < TIGHT


def test_capsule_layout():
    check_capsule_layout()


def check_replay_prefix():
    Hk, Hv, Dk, Dv, cap = 1, 2, 6, 4, 4
    lengths = [4, 3, 4, 0]
    inp = _tiny(lengths, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, seed=26, capacity=cap)
    _, _, capsule = _forward(inp, state_update_capacity=cap)
    cu = inp["cu_seqlens"]
    for m in range(cap + 1):
        accepted = np.array([min(m, L) for L in lengths])
        dst = O.gdn_replay(inp["initial_state"], capsule, accepted, Hk, Hv, Dk, Dv)
        # the recurrence on just the accepted prefix of every request
        sub = dict(inp)
        idx = np.concatenate([np.arange(cu[r], cu[r] + accepted[r]) for r in range(len(lengths))]).astype(int)
        for name in ("q", "k", "v", "a", "b"):
            sub[name] = inp[name][idx]
        sub["cu_seqlens"] = cu_from_lengths(accepted)
        _, fin_m, _ = _forward(sub)
        assert _rel(dst, fin_m) < TIGHT, m
        if m == 0:
            assert np.array_equal(dst, inp["initial_state"].astype(np.float64))


def test_replay_prefix():
    check_replay_prefix()


def check_capture_count_clamp():
    """capture_count beyond capacity captures capacity rows; below zero, none.

    The capture contract of the compact causal convolution ("[CUDA] Add compact
    GatedDeltaNet operator", embedded commit, Validation: capture-count
    requirements and capacity bounds), read the same way for the capsule. Rows
    are checked against the Householder brute force, not against the oracle."""
    Hk, Hv, Dk, Dv, cap = 1, 2, 6, 4, 3
    lengths = [6, 6, 2, 5]
    inp = _tiny(lengths, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, seed=29, capacity=cap)
    R = len(lengths)
    W = O.capsule_width(Hk, Hv, Dk, Dv)
    poison = np.full((R, cap, W), -7.25)
    counts = np.array([99, -5, 99, 2])
    _, _, capsule = _forward(inp, state_update_capacity=cap, capture_count=counts,
                             state_update_init=poison)
    _, _, full = _forward(inp, state_update_capacity=cap, state_update_init=poison)
    alpha, beta = bf.closed_form_gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    q, k, v = (inp[n].astype(np.float64) for n in ("q", "k", "v"))
    cu = inp["cu_seqlens"]
    expect_rows = [3, 0, 2, 2]                       # min(len, clamp(count, 0, cap))
    for r in range(R):
        t0, t1 = cu[r], cu[r + 1]
        n = expect_rows[r]
        assert np.all(capsule[r, n:] == -7.25)      # nothing past n_r, nothing at all for -5
        for h in range(Hv):
            _, _, deltas = bf.transition_form(q[t0:t1, 0], k[t0:t1, 0], v[t0:t1, h], alpha[t0:t1, h],
                                              beta[t0:t1, h], inp["initial_state"][r, h].astype(np.float64),
                                              1.0 / math.sqrt(Dk))
            d0 = Hv + Hk * Dk + h * Dv
            for j in range(n):
                assert _rel(capsule[r, j, d0:d0 + Dv], deltas[j]) < TIGHT
                assert abs(capsule[r, j, h] - alpha[t0 + j, h]) <= 1e-13 * alpha[t0 + j, h]
    # a count of 99 is the same capture as no counts at all (capacity rows)
    assert np.array_equal(capsule[0], full[0]) and np.array_equal(capsule[2], full[2])


def test_capture_count_clamp():
    check_capture_count_clamp()


def check_replay_accepted_clamp():
    """accepted beyond capacity replays the capacity rows; below zero, none (a copy).

    Checked against the recurrence run on the clamped prefix of each request
    (P-9) and, for the copy, against the committed state itself."""
    Hk, Hv, Dk, Dv, cap = 1, 2, 6, 4, 3
    lengths = [5, 4, 3]
    inp = _tiny(lengths, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, seed=30, capacity=cap)
    _, _, capsule = _forward(inp, state_update_capacity=cap)
    cu = inp["cu_seqlens"]
    accepted = np.array([99, -3, 3])
    dst = O.gdn_replay(inp["initial_state"], capsule, accepted, Hk, Hv, Dk, Dv)
    m = [3, 0, 3]
    sub = dict(inp)
    idx = np.concatenate([np.arange(cu[r], cu[r] + m[r]) for r in range(len(lengths))]).astype(int)
    for name in ("q", "k", "v", "a", "b"):
        sub[name] = inp[name][idx]
    sub["cu_seqlens"] = cu_from_lengths(m)
    _, fin_m, _ = _forward(sub)
    assert _rel(dst, fin_m) < TIGHT
    assert np.array_equal(dst[1], inp["initial_state"][1].astype(np.float64))


def test_replay_accepted_clamp():
    check_replay_accepted_clamp()


# ----------------------------------------------- P-10 packing invariance
def check_packing_invariance():
    with open(os.path.join(GOLDEN, "ragged_prompt_lengths.json")) as f:
        lengths = json.load(f)["lengths"]                         # 17, 512, 1993
    scaled = [max(1, L // 40) for L in lengths] + [0]             # same ragged mix, small
    inp = _tiny(scaled, Hk=1, Hv=2, Dk=6, Dv=4, seed=27)
    out, fin, _ = _forward(inp)
    cu = inp["cu_seqlens"]
    for r in range(len(scaled)):
        sub = dict(inp)
        for name in ("q", "k", "v", "a", "b"):
            sub[name] = inp[name][cu[r]:cu[r + 1]]
        sub["cu_seqlens"] = cu_from_lengths([scaled[r]])
        sub["initial_state"] = inp["initial_state"][r:r + 1]
        o1, f1, _ = _forward(sub)
        assert np.array_equal(o1, out[cu[r]:cu[r + 1]]) and np.array_equal(f1[0], fin[r])


def test_packing_invariance():
    check_packing_invariance()


def test_zero_length_segments_keep_state():
    inp = _tiny([0, 3, 0], Hk=1, Hv=1, Dk=4, Dv=3, seed=28)
    out, fin, _ = _forward(inp)
    assert np.array_equal(fin[0], inp["initial_state"][0]) and np.array_equal(fin[2], inp["initial_state"][2])
    inp0 = _tiny([0, 2], Hk=1, Hv=1, Dk=4, Dv=3, seed=28, initial="zero")
    _, fin0, _ = _forward(inp0)
    assert np.all(fin0[0] == 0)


# ------------------------------------------------------------ P-11 GQA
def check_gqa():
    Hk, Hv = 2, 6
    inp = _tiny([5, 3], Hk=Hk, Hv=Hv, Dk=5, Dv=4, seed=29)
    out, fin, _ = _forward(inp)
    mha = dict(inp)
    G = Hv // Hk
    mha["q"] = np.repeat(inp["q"], G, axis=1)                     # value head h reads key head h // G
    mha["k"] = np.repeat(inp["k"], G, axis=1)
    o2, f2, _ = _forward(mha)
    assert np.array_equal(out, o2) and np.array_equal(fin, f2)
    # with Hk = Hv every head runs alone
    for h in range(Hv):
        one = dict(mha)
        for name in ("q", "k", "v"):
            one[name] = mha[name][:, h:h + 1]
        for name in ("a", "b"):
            one[name] = mha[name][:, h:h + 1]
        one["A_log"], one["dt_bias"] = mha["A_log"][h:h + 1], mha["dt_bias"][h:h + 1]
        one["initial_state"] = mha["initial_state"][:, h:h + 1]
        o1, f1, _ = _forward(one)
        assert np.array_equal(o1[:, 0], out[:, h]) and np.array_equal(f1[:, 0], fin[:, h])


def test_gqa():
    check_gqa()


# ------------------------------------------------------- P-12 geometry
def test_dense_checkpoint_geometry():
    with open(os.path.join(GOLDEN, "qwen38_dense_checkpoints.json")) as f:
        g = json.load(f)
    from gdn_workloads import WORKLOADS
    for name in ("spec_verify_replay", "long_prefill"):
        w = WORKLOADS[name]
        per_layer = w.Hv * w.Dv * w.Dk * g["state_dtype_bytes"]
        assert g["slots"] * g["gdn_layers"] * per_layer == g["dense_checkpoint_mib"] * 2 ** 20
    # the capsule that replaces them (decay, key, delta per token) is far smaller
    w = WORKLOADS["spec_verify_replay"]
    capsule_bytes = O.capsule_width(w.Hk, w.Hv, w.Dk, w.Dv) * 4
    assert capsule_bytes == 32960
    assert g["slots"] * g["gdn_layers"] * capsule_bytes * 90 < g["dense_checkpoint_mib"] * 2 ** 20


def test_workload_lengths_seeded():
    from gdn_workloads import workload_inputs
    inp = workload_inputs("tiny_recurrent")
    assert inp["q"].shape == (16, 2, 16) and inp["initial_state"] is None
    lens = make_inputs(None, 1, 1, 4, 4, "f16", 3, num_drawn=8, max_drawn=4096)["lengths"]
    assert list(lens) == [3324, 351, 735, 970, 743, 3283, 3561, 2385]


ALL_CHECKS = [
    check_gate_closed_form, check_normalisation, check_frozen_state, check_decay_only,
    check_exact_write, check_transition_form, check_materialised_form,
    check_chunked_equals_recurrent, check_capsule_layout, check_replay_prefix,
    check_packing_invariance, check_gqa, check_capture_count_clamp, check_replay_accepted_clamp,
]


# ------------------------------------------- effective gates (activation none)
def _effective(inp, alpha, beta):
    """The inputs with a, b replaced by effective gates; A_log, dt_bias unused."""
    e = dict(inp)
    e["a"] = np.asarray(alpha, np.float32)
    e["b"] = np.asarray(beta, np.float32)
    e["A_log"] = e["dt_bias"] = None
    return e


def test_effective_gates_frozen_state():
    # alpha = 1, beta = 0 passed as effective gates: the state stays frozen and
    # o_t = S0 q^_t with q^ = q / |q| * Dk^-1/2 written out here
    inp = _tiny([5, 3], Hk=1, Hv=2, Dk=6, Dv=4)
    e = _effective(inp, np.ones_like(inp["a"]), np.zeros_like(inp["b"]))
    out, fin, _ = _forward(e, gate_activation="none")
    assert np.array_equal(fin, inp["initial_state"].astype(np.float64))
    q = inp["q"].astype(np.float64)
    qh = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6) / np.sqrt(6)
    cu = inp["cu_seqlens"]
    for r in range(2):
        for t in range(cu[r], cu[r + 1]):
            for h in range(2):
                want = inp["initial_state"][r, h].astype(np.float64) @ qh[t, 0]
                assert np.allclose(out[t, h], want, rtol=0, atol=1e-12)


def test_effective_gates_decay_only():
    # beta = 0: S_T = prod_t alpha_t * S0 for the given alpha
    inp = _tiny([7], Hk=1, Hv=2, Dk=5, Dv=4)
    rng = np.random.default_rng(5)
    alpha = rng.uniform(0.2, 1.0, inp["a"].shape)
    e = _effective(inp, alpha, np.zeros_like(inp["b"]))
    _, fin, _ = _forward(e, gate_activation="none")
    gamma = np.prod(e["a"].astype(np.float64), axis=0)
    assert _rel(fin[0], gamma[:, None, None] * inp["initial_state"][0]) < TIGHT


def test_effective_gates_exact_write():
    # alpha = 1, beta = 1, orthonormal keys through the whole forward: S_n k_i = v_i
    rng = np.random.default_rng(6)
    Dk, Dv, n = 8, 5, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    inp = _tiny([n], Hk=1, Hv=1, Dk=Dk, Dv=Dv)
    inp["k"] = Qm[:, :n].T[:, None, :].astype(np.float64)
    e = _effective(inp, np.ones_like(inp["a"]), np.ones_like(inp["b"]))
    _, fin, _ = _forward(e, gate_activation="none")
    # exact up to the norm epsilon: |k^|^2 = 1 / (1 + 1e-6)
    for i in range(n):
        assert np.allclose(fin[0, 0] @ Qm[:, i], inp["v"][i, 0], rtol=0, atol=1e-5)


def test_effective_decay_is_clamped():
    # a decay above 1 acts as 1; one below 0 acts as 0, which resets the state:
    # after it S = beta v k^^T whatever S0 was
    inp = _tiny([1], Hk=1, Hv=1, Dk=4, Dv=3)
    beta = np.full_like(inp["b"], 0.5)
    over = _forward(_effective(inp, np.full_like(inp["a"], 1.7), beta), gate_activation="none")
    one = _forward(_effective(inp, np.ones_like(inp["a"]), beta), gate_activation="none")
    assert np.array_equal(over[1], one[1])
    _, fin, _ = _forward(_effective(inp, np.full_like(inp["a"], -0.3), beta), gate_activation="none")
    k = inp["k"][0, 0].astype(np.float64)
    kh = k / np.sqrt(k @ k + 1e-6)
    want = 0.5 * np.outer(inp["v"][0, 0].astype(np.float64), kh)
    assert np.allclose(fin[0, 0], want, rtol=0, atol=1e-12)


def test_dense_layout_is_uniform_packing():
    # the rank-4 layout [R, S, H, D] is the packed layout with offsets 0, S, 2S, ...
    inp = _tiny([4, 4, 4], Hk=1, Hv=2, Dk=4, Dv=3)
    assert np.array_equal(O.dense_cu_seqlens(12, 3), [0, 4, 8, 12])
    packed = _forward(inp)
    dense = O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                          inp["dt_bias"], None, inp["initial_state"], num_reqs=3)
    for x, y in zip(packed[:2], dense[:2]):
        assert np.array_equal(x, y)
    with pytest.raises(ValueError):
        O.dense_cu_seqlens(10, 3)
