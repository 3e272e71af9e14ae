"""Pins of the K-major layout oracle (oracle/layout_oracle.py): the gated delta
rule written out directly in K-major orientation (M = S^T, first page, Copilot
review: dense K-major [B, heads, key_dim, value_dim] against packed V-major
[B, heads, value_dim, key_dim]) on tiny inputs, with Dk != Dv so that a
transposed axis cannot go unnoticed."""
from __future__ import annotations

import numpy as np

from gdn_workloads import make_inputs
from oracle import gdn_oracle as GO
from oracle import layout_oracle as LO


def _k_major_by_hand(inp, M0, scale):
    """Token loop in K-major terms: u = beta (v - alpha M^T k^), M = alpha M + k^ u^T, o = M^T q^."""
    q, k, v = (np.asarray(inp[n], np.float64) for n in ("q", "k", "v"))
    N, Hk, Dk = q.shape
    Hv = v.shape[1]
    alpha, beta = GO.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    M = np.array(M0, np.float64, copy=True)
    out = np.zeros((N, Hv, v.shape[2]))
    for r in range(len(cu) - 1):
        for t in range(cu[r], cu[r + 1]):
            for h in range(Hv):
                g = h // (Hv // Hk)
                kh = k[t, g] / np.sqrt(k[t, g] @ k[t, g] + GO.L2NORM_EPS)
                qh = q[t, g] / np.sqrt(q[t, g] @ q[t, g] + GO.L2NORM_EPS) * scale
                Mh = M[r, h]                                        # [Dk, Dv]
                u = beta[t, h] * (v[t, h] - alpha[t, h] * (Mh.T @ kh))
                M[r, h] = alpha[t, h] * Mh + np.outer(kh, u)
                out[t, h] = M[r, h].T @ qh
    return out, M


def test_k_major_forward_matches_the_rule_written_in_k_major():
    inp = make_inputs([3, 0, 5], 1, 2, 6, 4, "f32", seed=31)
    M0 = np.random.default_rng(0).standard_normal((3, 2, 6, 4)) * 0.1
    o, M, _ = LO.gdn_forward_k_major(*[inp[n] for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                        "cu_seqlens")], M0)
    o_ref, M_ref = _k_major_by_hand(inp, M0, 1 / np.sqrt(6))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(M, M_ref, rtol=1e-12, atol=1e-14)
    assert M.shape == (3, 2, 6, 4)


def test_k_major_replay_is_the_prefix_forward():
    inp = make_inputs([4, 4], 1, 2, 6, 4, "f32", seed=32, capacity=4)
    M0 = np.random.default_rng(1).standard_normal((2, 2, 6, 4)) * 0.1
    args = [inp[n] for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")]
    _, _, cap = LO.gdn_forward_k_major(*args, M0, state_update_capacity=4)
    acc = np.array([3, 1])
    got = LO.gdn_replay_k_major(M0, cap, acc, 1, 2, 6, 4)
    for r in range(2):
        sub = make_inputs([4, 4], 1, 2, 6, 4, "f32", seed=32, capacity=4)
        t0 = int(sub["cu_seqlens"][r])
        m = int(acc[r])
        part = {n: sub[n][t0:t0 + m] for n in ("q", "k", "v", "a", "b")}
        part.update(A_log=sub["A_log"], dt_bias=sub["dt_bias"], cu_seqlens=np.array([0, m]))
        _, M_ref = _k_major_by_hand(part, M0[r:r + 1], 1 / np.sqrt(6))
        np.testing.assert_allclose(got[r], M_ref[0], rtol=1e-12, atol=1e-14)
