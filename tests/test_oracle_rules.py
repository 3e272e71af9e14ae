"""Pins of the oracle's update rules other than the gated delta rule.

The rules are read as the family the name gated_delta composes (the decay gate
and the delta correction each on or off); see oracle/gdn_oracle.py. No page
prints them or a worked example, so their absolute values are parity unpinned
against the pages; each is pinned here against a formula written out
independently of the oracle (materialised attention with explicit decay
products, the Householder transition-matrix form, exact writes on orthonormal
keys), and the chunked form and the capsule replay against the recurrence for
every rule. Planted mistakes at the end check that the pins catch errors in
the code paths these rules add.
"""
from __future__ import annotations

import math
import warnings

import numpy as np
import pytest

import brute_force as bf
from gdn_workloads import cu_from_lengths, make_inputs
from oracle import gdn_oracle as O

TIGHT = 1e-11
RULES = ["gated_delta", "delta", "gated", "linear"]


def _rel(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-300))


def _inputs(lengths, Hk=1, Hv=2, Dk=6, Dv=5, seed=31, capacity=0):
    return make_inputs(lengths, Hk, Hv, Dk, Dv, "f32", seed, capacity=capacity)


def _forward(inp, rule, **kw):
    gated, delta = O.rule_parts(rule)
    # inputs a rule does not read are passed as None
    return O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"] if gated else None,
                         inp["b"] if delta else None, inp["A_log"] if gated else None,
                         inp["dt_bias"] if gated else None, inp["cu_seqlens"], inp["initial_state"],
                         update_rule=rule, **kw)


def _attention(q, k, v, alpha, S0, scale):
    """Materialised (gated) linear attention of one sequence and head, decays as
    explicit products: o_t = gamma_t S0 q^_t + sum_{i<=t} (gamma_t / gamma_i)
    (k^_i . q^_t) v_i; S_T = gamma_T S0 + sum_i (gamma_T / gamma_i) v_i k^_i^T."""
    T = k.shape[0]
    K = [bf.unit(k[t]) for t in range(T)]
    Q = [bf.unit(q[t]) * scale for t in range(T)]

    def decay(t, i):                                   # prod_{j=i+1..t} alpha_j
        p = 1.0
        for j in range(i + 1, t + 1):
            p *= float(alpha[j])
        return p

    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        acc = decay(t, -1) * (S0 @ Q[t])
        for i in range(t + 1):
            acc = acc + decay(t, i) * float(K[i] @ Q[t]) * v[i]
        o[t] = acc
    S = decay(T - 1, -1) * np.array(S0, np.float64)
    for i in range(T):
        S = S + decay(T - 1, i) * np.outer(v[i], K[i])
    return o, S


def _per_head(inp, rule, form):
    alpha, beta = bf.closed_form_gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    gated, delta = O.rule_parts(rule)
    if not gated:
        alpha = np.ones_like(alpha)
    q, k, v = (inp[n].astype(np.float64) for n in ("q", "k", "v"))
    cu = inp["cu_seqlens"]
    Hv, Dk = inp["Hv"], q.shape[2]
    G = Hv // inp["Hk"]
    out = np.zeros(v.shape)
    fin = np.zeros(inp["initial_state"].shape)
    for r in range(len(cu) - 1):
        t0, t1 = cu[r], cu[r + 1]
        for h in range(Hv):
            S0 = inp["initial_state"][r, h].astype(np.float64)
            if t1 == t0:
                fin[r, h] = S0
                continue
            args = (q[t0:t1, h // G], k[t0:t1, h // G], v[t0:t1, h])
            if form == "attention":
                o, S = _attention(*args, alpha[t0:t1, h], S0, 1.0 / math.sqrt(Dk))
            else:
                o, states, _ = bf.transition_form(*args, alpha[t0:t1, h], beta[t0:t1, h], S0, 1.0 / math.sqrt(Dk))
                S = states[-1]
            out[t0:t1, h] = o
            fin[r, h] = S
    return out, fin


def check_linear_rule_is_causal_linear_attention():
    inp = _inputs([7, 0, 4], seed=32)
    o, s, _ = _forward(inp, "linear")
    ref_o, ref_s = _per_head(inp, "linear", "attention")
    assert _rel(o, ref_o) < TIGHT and _rel(s, ref_s) < TIGHT


def test_linear_rule_is_causal_linear_attention():
    check_linear_rule_is_causal_linear_attention()


def check_gated_rule_is_decayed_attention():
    inp = _inputs([6, 5], Hk=1, Hv=2, seed=33)
    o, s, _ = _forward(inp, "gated")
    ref_o, ref_s = _per_head(inp, "gated", "attention")
    assert _rel(o, ref_o) < TIGHT and _rel(s, ref_s) < TIGHT


def test_gated_rule_is_decayed_attention():
    check_gated_rule_is_decayed_attention()


def check_delta_rule_is_householder_form():
    # DeltaNet: S_t = S_{t-1} (I - beta k^ k^^T) + beta v k^^T, the transition form with alpha = 1
    inp = _inputs([5, 3], Hk=1, Hv=2, seed=34)
    o, s, _ = _forward(inp, "delta")
    ref_o, ref_s = _per_head(inp, "delta", "householder")
    assert _rel(o, ref_o) < TIGHT and _rel(s, ref_s) < TIGHT


def test_delta_rule_is_householder_form():
    check_delta_rule_is_householder_form()


def check_delta_rule_exact_write():
    # beta = 1 (effective gates) on orthonormal keys: every key reads back its value,
    # the orthogonal complement keeps the initial state
    rng = np.random.default_rng(35)
    Dk, Dv, n = 8, 5, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:, :n].T
    inp = {"q": rng.standard_normal((n, 1, Dk)), "k": keys[:, None, :] * 3.0, "v": rng.standard_normal((n, 1, Dv)),
           "b": np.ones((n, 1)), "S0": rng.standard_normal((1, 1, Dv, Dk))}
    _, S, _ = O.gdn_forward(inp["q"], inp["k"], inp["v"], None, inp["b"], None, None, [0, n], inp["S0"],
                            gate_activation="none", update_rule="delta")
    for i in range(n):
        assert np.allclose(S[0, 0] @ keys[i], inp["v"][i, 0], rtol=0, atol=1e-6)   # eps of the norm
    for x in Qm[:, n:].T:
        assert np.allclose(S[0, 0] @ x, inp["S0"][0, 0] @ x, rtol=0, atol=1e-12)


def test_delta_rule_exact_write():
    check_delta_rule_exact_write()


def check_chunked_equals_recurrent_every_rule():
    inp = _inputs([70, 1, 0, 130], Hk=1, Hv=2, seed=36)
    for rule in RULES:
        o, s, _ = _forward(inp, rule)
        gated, delta = O.rule_parts(rule)
        for c in (1, 7, 64):
            oc, sc = O.chunked_forward(inp["q"], inp["k"], inp["v"], inp["a"] if gated else None,
                                       inp["b"] if delta else None, inp["A_log"] if gated else None,
                                       inp["dt_bias"] if gated else None, inp["cu_seqlens"],
                                       inp["initial_state"], chunk=c, update_rule=rule)
            assert _rel(oc, o) < 1e-10 and _rel(sc, s) < 1e-10, (rule, c)


def test_chunked_equals_recurrent_every_rule():
    check_chunked_equals_recurrent_every_rule()


def check_capsule_replay_every_rule():
    # S_t = alpha_t S_{t-1} + u_t k^_t^T holds for every rule (u = v and alpha = 1 where
    # the rule has no delta or no gate): replaying m rows equals m tokens of the recurrence
    Hk, Hv, Dk, Dv, cap = 1, 2, 6, 4, 4
    lengths = [4, 3, 4]
    inp = _inputs(lengths, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, seed=37, capacity=cap)
    cu = inp["cu_seqlens"]
    for rule in RULES:
        gated, delta = O.rule_parts(rule)
        _, _, capsule = _forward(inp, rule, state_update_capacity=cap)
        alpha_sec = capsule[:, :, :Hv]
        if not gated:
            assert np.all(alpha_sec[0, :4] == 1.0) and np.all(alpha_sec[1, :3] == 1.0)
        for m in range(cap + 1):
            acc = np.array([min(m, L) for L in lengths])
            dst = O.gdn_replay(inp["initial_state"], capsule, acc, Hk, Hv, Dk, Dv)
            sub = dict(inp)
            idx = np.concatenate([np.arange(cu[r], cu[r] + acc[r]) for r in range(len(lengths))]).astype(int)
            for name in ("q", "k", "v", "a", "b"):
                sub[name] = inp[name][idx]
            sub["cu_seqlens"] = cu_from_lengths(acc)
            _, fin_m, _ = _forward(sub, rule)
            assert _rel(dst, fin_m) < TIGHT, (rule, m)


def test_capsule_replay_every_rule():
    check_capsule_replay_every_rule()


def test_unknown_rule_is_refused():
    with pytest.raises(ValueError):
        O.rule_parts("gated_linear")


RULE_CHECKS = [check_linear_rule_is_causal_linear_attention, check_gated_rule_is_decayed_attention,
               check_delta_rule_is_householder_form, check_delta_rule_exact_write,
               check_chunked_equals_recurrent_every_rule, check_capsule_replay_every_rule]


# ------------------------------------------------------------ planted mistakes
def _any_rule_check_fails():
    failed = []
    for check in RULE_CHECKS:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore", RuntimeWarning)
                check()
        except Exception:
            failed.append(check.__name__)
    return failed


def _plain_variant(kind):
    def rec(qh, kh, v, alpha, S0):
        T, H, Dv = v.shape
        S = np.array(S0, dtype=np.float64, copy=True)
        o = np.zeros((T, H, Dv))
        for t in range(T):
            S_prev = S
            a_t = np.ones_like(alpha[t]) if kind == "no_decay" else alpha[t]
            S = a_t[:, None, None] * S + v[t][:, :, None] * kh[t][:, None, :]
            o[t] = np.einsum("hvk,hk->hv", S_prev if kind == "old_state" else S, qh[t])
        return o, S, np.array(v, dtype=np.float64, copy=True)
    return rec


@pytest.mark.parametrize("kind", ["no_decay", "old_state"])
def test_plain_write_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(O, "plain_write_recurrence", _plain_variant(kind))
    assert _any_rule_check_fails(), kind


def test_plain_chunk_without_key_decay_is_caught(monkeypatch):
    def step(qh, kh, v, log_alpha, S0):
        L, H, Dk = kh.shape
        o = np.zeros((L, H, v.shape[2]))
        S_out = np.zeros((H, v.shape[2], Dk))
        g = np.cumsum(log_alpha, axis=0)
        incl = np.tril(np.ones((L, L), dtype=bool), 0)
        for h in range(H):
            K, Q, V, gh = kh[:, h], qh[:, h], v[:, h], g[:, h]
            M = np.exp(np.where(incl, gh[:, None] - gh[None, :], -np.inf))
            o[:, h] = np.exp(gh)[:, None] * (Q @ S0[h].T) + (M * (Q @ K.T)) @ V
            S_out[h] = np.exp(gh[-1]) * S0[h] + V.T @ K           # key decay dropped
        return o, S_out
    monkeypatch.setattr(O, "chunk_step_plain_write", step)
    assert "check_chunked_equals_recurrent_every_rule" in _any_rule_check_fails()


def test_rule_parts_swapped_is_caught(monkeypatch):
    # the gate and delta switches read the wrong way round
    monkeypatch.setattr(O, "rule_parts", lambda rule: (rule in ("gated_delta", "delta"),
                                                       rule in ("gated_delta", "gated")))
    assert _any_rule_check_fails()
