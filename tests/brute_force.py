"""Brute-force reformulations of the gated delta rule, for tiny inputs only.

These pin the float64 oracle to something other than itself. They share no
code with it and use different (mathematically equivalent) formulas:

* gates from the closed form alpha = (1 + e^x)^(-exp(A_log)) in pure Python;
* the state recurrence as a product of explicit Dk x Dk transition matrices,
  S_t = S_{t-1} alpha_t (I - beta_t k^ k^^T) + beta_t v_t k^^T (the generalised
  Householder form of the delta rule);
* the materialised (parallel) form, in which every decay between two tokens is
  an explicit product of alphas and the deltas solve one unit-lower-triangular
  system with scipy's triangular solver.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.linalg import solve_triangular


def closed_form_gates(a, b, A_log, dt_bias):
    """alpha = (1 + e^x)^(-A), A = e^{A_log}; beta = 1 / (1 + e^-b); per element in Python."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    alpha = np.empty_like(a)
    beta = np.empty_like(b)
    for idx in np.ndindex(a.shape):
        h = idx[-1]
        x = float(a[idx]) + float(dt_bias[h])
        A = math.exp(float(A_log[h]))
        if x > 30.0:          # (1 + e^x)^-A = e^{-A x} (1 + e^-x)^-A, no overflow
            alpha[idx] = math.exp(-A * x) * math.pow(1.0 + math.exp(-x), -A)
        else:
            alpha[idx] = math.pow(1.0 + math.exp(x), -A)
        beta[idx] = 1.0 / (1.0 + math.exp(-float(b[idx])))
    return alpha, beta


def unit(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / math.sqrt(float(np.dot(x, x)) + eps)


def transition_form(q, k, v, alpha, beta, S0, scale):
    """One sequence, one head. q, k [T, Dk]; v [T, Dv]; alpha, beta [T]; S0 [Dv, Dk].

    Returns (o [T, Dv], states [T, Dv, Dk], deltas [T, Dv]).
    """
    T, Dk = k.shape
    S = np.array(S0, np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    states = np.zeros((T,) + S.shape)
    deltas = np.zeros((T, v.shape[1]))
    I = np.eye(Dk)
    for t in range(T):
        kh = unit(k[t])
        qh = unit(q[t]) * scale
        deltas[t] = beta[t] * (v[t] - alpha[t] * (S @ kh))
        S = S @ (alpha[t] * (I - beta[t] * np.outer(kh, kh))) + beta[t] * np.outer(v[t], kh)
        states[t] = S
        o[t] = S @ qh
    return o, states, deltas


def materialised_form(q, k, v, alpha, beta, S0, scale):
    """Parallel form over the whole sequence (one head), explicit decay products.

    decay(t, i) = prod_{j=i+1..t} alpha_j; gamma_t = prod_{j<=t} alpha_j.
    (I + A) u = beta (v - gamma S0 k^), A[t, i] = beta_t decay(t, i) k^_t.k^_i (i < t);
    o_t = gamma_t S0 q^_t + sum_{i<=t} decay(t, i) (q^_t . k^_i) u_i;
    S_T = gamma_{T-1} S0 + sum_i decay(T-1, i) u_i k^_i^T.
    """
    T = k.shape[0]
    K = np.stack([unit(k[t]) for t in range(T)])
    Q = np.stack([unit(q[t]) * scale for t in range(T)])

    def decay(t, i):
        p = 1.0
        for j in range(i + 1, t + 1):
            p *= float(alpha[j])
        return p

    gamma = [decay(t, -1) for t in range(T)]
    A = np.zeros((T, T))
    rhs = np.zeros((T, v.shape[1]))
    for t in range(T):
        for i in range(t):
            A[t, i] = beta[t] * decay(t, i) * float(K[t] @ K[i])
        rhs[t] = beta[t] * (v[t] - gamma[t] * (S0 @ K[t]))
    u = solve_triangular(np.eye(T) + A, rhs, lower=True, unit_diagonal=True)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        acc = gamma[t] * (S0 @ Q[t])
        for i in range(t + 1):
            acc = acc + decay(t, i) * float(Q[t] @ K[i]) * u[i]
        o[t] = acc
    S = gamma[T - 1] * np.array(S0, np.float64)
    for i in range(T):
        S = S + decay(T - 1, i) * np.outer(u[i], K[i])
    return o, S, u
