"""Plain float64 reference of the K-major state layout.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the operator library.

The first page's Copilot review notes that the two recurrent-state layouts of
the exporter differ: the packed GatedDeltaNet path keeps a V-major state
[B, heads, value_dim, key_dim] and the dense LinearAttention path a K-major one
[B, heads, key_dim, value_dim]. Both hold the same matrix; K-major stores its
transpose, M = S^T, so in K-major terms the gated delta rule reads

  u_t = beta_t (v_t - alpha_t M^T k^_t),  M_t = alpha_t M_{t-1} + k^_t u_t^T,  o_t = M_t^T q^_t.

A K-major call is the V-major oracle between transposes of the state's last
two axes.
"""
from __future__ import annotations

import numpy as np

from . import gdn_oracle as GO


def to_k_major(state):
    """[..., Dv, Dk] V-major -> [..., Dk, Dv] K-major (or back: the map is its own inverse)."""
    return None if state is None else np.swapaxes(np.asarray(state, np.float64), -1, -2)


def gdn_forward_k_major(q, k, v, a, b, A_log, dt_bias, cu_seqlens, initial_state=None, **kw):
    """gdn_forward with the initial and final states K-major [R, Hv, Dk, Dv]."""
    o, S, cap = GO.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, to_k_major(initial_state), **kw)
    return o, to_k_major(S), cap


def gdn_replay_k_major(src_state, state_update, accepted, Hk, Hv, Dk, Dv):
    """gdn_replay with K-major states [R, Hv, Dk, Dv]."""
    return to_k_major(GO.gdn_replay(to_k_major(src_state), state_update, accepted, Hk, Hv, Dk, Dv))
