"""Plain float64 reference of the pooled fixed-state banks.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the operator library.

"Replay compact fixed state for hybrid decoding" (Key Changes; Copilot
overview) keeps each request's fixed recurrent state - the GatedDeltaNet state
and the causal-convolution state - in a fixed-state pool with per-request
ownership and double-buffered publication: a speculative step verifies against
the committed bank, replays the accepted prefix into the inactive bank, and
publishes that bank. Written out for a pool of P slots and per-request slot
indices:

  gather(pool, slots)[r]  = pool[slots[r]] if 0 <= slots[r] < P, else a zero state
  scatter(pool, slots, S) : pool[slots[r]] = S[r] for every r with 0 <= slots[r] < P;
                            every other slot keeps its contents
  publish(committed, inactive) = (inactive, committed)     the two slot lists trade places

A pooled call is the request-indexed call of gdn_oracle / conv_oracle between
a gather of the read slots and a scatter to the write slots. A missing slot
list means slot r for request r.
"""
from __future__ import annotations

import numpy as np

from . import conv_oracle as CO
from . import gdn_oracle as GO


def _slots(slots, R):
    return np.arange(R, dtype=np.int64) if slots is None else np.asarray(slots, np.int64)


def gather(pool, slots, R, state_shape):
    """States [R, *state_shape] read from `pool` ([P, *state_shape] or None)."""
    out = np.zeros((R,) + tuple(state_shape))
    if pool is None:
        return out
    pool = np.asarray(pool, np.float64)
    P = pool.shape[0]
    for r, s in enumerate(_slots(slots, R)):
        if 0 <= s < P:
            out[r] = pool[s]
    return out


def scatter(pool, slots, states):
    """A copy of `pool` with states[r] written to slot slots[r] where that slot exists."""
    out = np.array(pool, np.float64, copy=True)
    P = out.shape[0]
    for r, s in enumerate(_slots(slots, len(states))):
        if 0 <= s < P:
            out[s] = states[r]
    return out


def publish(committed, inactive):
    """Double-buffered publication: the slot lists trade places."""
    return np.array(inactive, copy=True), np.array(committed, copy=True)


def gdn_forward_pooled(q, k, v, a, b, A_log, dt_bias, cu_seqlens, pool, read_slots, write_slots,
                       out_pool=None, num_reqs=None, **kw):
    """GatedDeltaNet forward from and into pools [P, Hv, Dv, Dk]. `out_pool` is
    the write pool before the call (default: the read pool). Returns (output,
    write pool after the call, capsule or None)."""
    Hv, Dv = v.shape[1], v.shape[2]
    Dk = k.shape[2]
    R = (len(cu_seqlens) - 1) if cu_seqlens is not None else num_reqs
    S0 = gather(pool, read_slots, R, (Hv, Dv, Dk))
    o, S1, cap = GO.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, S0, num_reqs=num_reqs, **kw)
    base = pool if out_pool is None else out_pool
    return o, scatter(base, write_slots, S1), cap


def gdn_replay_pooled(pool, state_update, accepted, read_slots, write_slots, Hk, Hv, Dk, Dv,
                      out_pool=None):
    """GatedDeltaNet replay from and into pools; returns the write pool after the call."""
    R = len(accepted)
    src = gather(pool, read_slots, R, (Hv, Dv, Dk))
    dst = GO.gdn_replay(src, state_update, accepted, Hk, Hv, Dk, Dv)
    return scatter(pool if out_pool is None else out_pool, write_slots, dst)


def conv_forward_pooled(x, weight, bias, cu_seqlens, pool, read_slots, write_slots, out_pool=None,
                        num_reqs=None, **kw):
    """Causal convolution forward from and into pools [P, C, K - 1]. Returns
    (output, write pool after the call, capture or None)."""
    C, K = np.asarray(weight).shape
    R = (len(cu_seqlens) - 1) if cu_seqlens is not None else num_reqs
    s0 = gather(pool, read_slots, R, (C, K - 1))
    out, fin, cap = CO.conv_forward(x, weight, bias, cu_seqlens, s0, num_reqs=num_reqs, **kw)
    base = pool if out_pool is None else out_pool
    return out, scatter(base, write_slots, fin), cap


def conv_replay_pooled(pool, state_update, accepted, read_slots, write_slots, out_pool=None):
    """Causal convolution replay from and into pools; returns the write pool after the call."""
    pool = np.asarray(pool, np.float64)
    R = len(accepted)
    src = gather(pool, read_slots, R, pool.shape[1:])
    dst = CO.conv_replay(src, state_update, accepted)
    return scatter(pool if out_pool is None else out_pool, write_slots, dst)
