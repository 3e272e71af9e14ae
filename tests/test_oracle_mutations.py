"""Plant plausible mistakes in the float64 oracle (on the CPU only) and check
that at least one pin in test_oracle_pins catches each of them."""
from __future__ import annotations

import warnings

import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import gdn_oracle as O


def _any_check_fails():
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore", RuntimeWarning)
                check()
        except Exception:                                    # assertion or a crash
            failed.append(check.__name__)
    return failed


def _recurrence_variant(kind):
    def rec(qh, kh, v, alpha, beta, S0):
        T, H, Dv = v.shape
        S = np.array(S0, dtype=np.float64, copy=True)
        o = np.zeros((T, H, Dv))
        u_all = np.zeros((T, H, Dv))
        for t in range(T):
            a_t = alpha[t][:, None]
            Sk = np.einsum("hvk,hk->hv", S, kh[t])
            if kind == "delta_without_decay":
                u = beta[t][:, None] * (v[t] - Sk)
            elif kind == "delta_sign":
                u = beta[t][:, None] * (v[t] + a_t * Sk)
            else:
                u = beta[t][:, None] * (v[t] - a_t * Sk)
            S_prev = S
            if kind == "no_decay_on_state":
                S = S + u[:, :, None] * kh[t][:, None, :]
            else:
                S = a_t[:, :, None] * S + u[:, :, None] * kh[t][:, None, :]
            if kind == "output_from_old_state":
                o[t] = np.einsum("hvk,hk->hv", S_prev, qh[t])
            elif kind == "output_reads_key":
                o[t] = np.einsum("hvk,hk->hv", S, kh[t])
            else:
                o[t] = np.einsum("hvk,hk->hv", S, qh[t])
            u_all[t] = u
        return o, S, u_all
    return rec


RECURRENCE_MUTANTS = ["delta_without_decay", "delta_sign", "no_decay_on_state",
                      "output_from_old_state", "output_reads_key"]


@pytest.mark.parametrize("kind", RECURRENCE_MUTANTS)
def test_recurrence_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(O, "recurrence", _recurrence_variant(kind))
    assert _any_check_fails(), kind


def test_softplus_sign_is_caught(monkeypatch):
    monkeypatch.setattr(O, "softplus", lambda x: np.maximum(-np.asarray(x, float), 0.0)
                        + np.log1p(np.exp(-np.abs(np.asarray(x, float)))))
    assert _any_check_fails()


def test_beta_sign_is_caught(monkeypatch):
    orig = O.gates

    def gates(a, b, A_log, dt_bias):
        al, _ = orig(a, b, A_log, dt_bias)
        return al, 1.0 / (1.0 + np.exp(np.asarray(b, float)))
    monkeypatch.setattr(O, "gates", gates)
    assert _any_check_fails()


def test_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(O, "key_head_index", lambda Hk, Hv: np.arange(Hv) % Hk)
    assert _any_check_fails()


def test_scale_on_key_is_caught(monkeypatch):
    def unit_qk(q, k, Hv, scale):
        Dk = q.shape[-1]
        s = Dk ** -0.5 if scale is None else scale
        g = O.key_head_index(q.shape[1], Hv)
        return O.l2normalize(q)[:, g, :] * s, O.l2normalize(k)[:, g, :] * s
    monkeypatch.setattr(O, "_unit_qk", unit_qk)
    assert _any_check_fails()


def test_missing_query_scale_is_caught(monkeypatch):
    def unit_qk(q, k, Hv, scale):
        g = O.key_head_index(q.shape[1], Hv)
        return O.l2normalize(q)[:, g, :], O.l2normalize(k)[:, g, :]
    monkeypatch.setattr(O, "_unit_qk", unit_qk)
    assert _any_check_fails()


def test_norm_without_sqrt_is_caught(monkeypatch):
    monkeypatch.setattr(O, "l2normalize", lambda x, eps=O.L2NORM_EPS: np.asarray(x, float)
                        / (np.sum(np.asarray(x, float) ** 2, axis=-1, keepdims=True) + eps))
    assert _any_check_fails()


def _chunk_variant(kind):
    from scipy.linalg import solve_triangular

    def step(qh, kh, v, log_alpha, beta, S0):
        L, H, Dk = kh.shape
        o = np.zeros((L, H, v.shape[2]))
        S_out = np.zeros((H, v.shape[2], Dk))
        g = np.cumsum(log_alpha, axis=0)
        strict = np.tril(np.ones((L, L), bool), 0 if kind == "diag_in_A" else -1)
        incl = np.tril(np.ones((L, L), bool), 0)
        for h in range(H):
            K, Q, V, gh, bh = kh[:, h], qh[:, h], v[:, h], g[:, h], beta[:, h]
            diff = gh[:, None] - gh[None, :]
            A = np.where(strict, bh[:, None] * np.exp(np.where(strict, diff, -np.inf)) * (K @ K.T), 0.0)
            rhs = bh[:, None] * (V - np.exp(gh)[:, None] * (K @ S0[h].T))
            # "diag_in_A" keeps beta_r (k^_r . k^_r) on the diagonal of I + A
            U = solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=(kind != "diag_in_A"))
            M = np.exp(np.where(incl, diff, -np.inf))
            first = (Q @ S0[h].T) if kind == "no_query_decay" else np.exp(gh)[:, None] * (Q @ S0[h].T)
            o[:, h] = first + (M * (Q @ K.T)) @ U
            tail = K if kind == "no_key_decay" else np.exp(gh[-1] - gh)[:, None] * K
            S_out[h] = np.exp(gh[-1]) * S0[h] + U.T @ tail
        return o, S_out
    return step


@pytest.mark.parametrize("kind", ["diag_in_A", "no_query_decay", "no_key_decay"])
def test_chunk_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(O, "chunk_step", _chunk_variant(kind))
    assert _any_check_fails(), kind


def test_replay_without_decay_is_caught(monkeypatch):
    def replay(src_state, state_update, accepted, Hk, Hv, Dk, Dv):
        src = np.asarray(src_state, float)
        s_alpha, s_key, s_delta = O.capsule_sections(Hk, Hv, Dk, Dv)
        g = O.key_head_index(Hk, Hv)
        dst = np.array(src, copy=True)
        for r in range(src.shape[0]):
            for j in range(int(accepted[r])):
                row = np.asarray(state_update, float)[r, j]
                kk = row[s_key].reshape(Hk, Dk)[g]
                uu = row[s_delta].reshape(Hv, Dv)
                dst[r] = dst[r] + uu[:, :, None] * kk[:, None, :]
        return dst
    monkeypatch.setattr(O, "gdn_replay", replay)
    assert _any_check_fails()


def test_capsule_section_order_is_caught(monkeypatch):
    def sections(Hk, Hv, Dk, Dv):                      # key before decay
        return (slice(Hk * Dk, Hk * Dk + Hv), slice(0, Hk * Dk),
                slice(Hv + Hk * Dk, Hv + Hk * Dk + Hv * Dv))
    monkeypatch.setattr(O, "capsule_sections", sections)
    assert _any_check_fails()


def test_replay_reading_past_capacity_is_caught(monkeypatch):
    # accepted taken as given: the replay reads rows the request does not own
    real = O.gdn_replay

    def replay(src_state, state_update, accepted, Hk, Hv, Dk, Dv):
        su = np.asarray(state_update, float)
        acc = np.asarray(accepted)
        grown = np.concatenate([su, np.zeros((su.shape[0], int(max(acc.max(), 0)), su.shape[2]))], axis=1)
        return real(src_state, grown, acc, Hk, Hv, Dk, Dv)
    monkeypatch.setattr(O, "gdn_replay", replay)
    assert "check_replay_accepted_clamp" in _any_check_fails()


def test_capture_count_without_clamp_is_caught(monkeypatch):
    # a negative count read as "capture everything"
    real = O.gdn_forward

    def forward(*args, capture_count=None, **kw):
        if capture_count is not None:
            cap = kw.get("state_update_capacity", 0)
            capture_count = np.where(np.asarray(capture_count) < 0, cap, capture_count)
        return real(*args, capture_count=capture_count, **kw)
    monkeypatch.setattr(O, "gdn_forward", forward)
    assert "check_capture_count_clamp" in _any_check_fails()
