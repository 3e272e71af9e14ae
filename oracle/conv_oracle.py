"""Plain float64 reference of the compact VarlenCausalConvWithState operator.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the operator library.

What is computed, and where it comes from
-----------------------------------------
The pages describe the convolution that sits directly upstream of the
GatedDeltaNet operator in every hybrid layer as a "fused depthwise conv1d +
SiLU + carry state" over dense [B, C, S] or packed token-major [num_tokens, C]
inputs ("Add GatedDeltaNet evaluation export for Qwen hybrid models", Copilot
review of the builder docstring), and its compact form as returning
[output, final_state, state_update] where state_update holds only "the
appended activation values" needed to replay an accepted speculative prefix,
shaped [batch_size, state_update_capacity, channels], with an optional
per-request capture_count; the full state is [channels, kernel_size - 1]
("[CUDA] Add compact GatedDeltaNet operator", the embedded VarlenCausalConv
commit, Description and Motivation). Written out per request r with the K - 1
carried inputs s (oldest first) and the request's L tokens x_0 .. x_{L-1}:

  e          = [s_0 .. s_{K-2}, x_0 .. x_{L-1}]          per channel c
  y_j[c]     = act(bias[c] + sum_{i<K} w[c, i] * e[j + i][c])   (x_j is e[j + K - 1])
  final[r]   = e[L .. L + K - 2]                          the last K - 1 inputs
  capture[r, j] = x_j  for j < n_r = min(L, capture_count[r] or capacity)
  replay(m)  = the last K - 1 of [s, capture[r, 0 .. m - 1]]

act is SiLU(z) = z / (1 + e^-z), or the identity. w is the depthwise filter in
the cross-correlation orientation of conv1d: w[c, K - 1] multiplies the newest
input. Everything is float64 on the exact values of the (possibly fp16-rounded)
inputs.
"""
from __future__ import annotations

import numpy as np


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def conv_forward(x, weight, bias, cu_seqlens, initial_state=None, activation="silu",
                 state_update_capacity=0, capture_count=None, state_update_init=None,
                 num_reqs=None):
    """Packed forward. x [N, C]; weight [C, K]; bias [C] or None; cu_seqlens
    [R + 1] (None: dense layout with num_reqs requests of N / R tokens);
    initial_state [R, C, K - 1] or None for zeros. Returns (output [N, C],
    final_state [R, C, K - 1], state_update [R, capacity, C] or None); capture
    rows from n_r on keep state_update_init (zeros by default)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(weight, np.float64)
    N, C = x.shape
    K = w.shape[1]
    if cu_seqlens is None:
        if not num_reqs or N % num_reqs:
            raise ValueError("the dense layout needs N divisible by R")
        cu = np.arange(num_reqs + 1, dtype=np.int64) * (N // num_reqs)
    else:
        cu = np.asarray(cu_seqlens, np.int64)
    R = cu.shape[0] - 1
    b = np.zeros(C) if bias is None else np.asarray(bias, np.float64)
    out = np.zeros((N, C))
    final = np.zeros((R, C, K - 1))
    cap = int(state_update_capacity)
    capture = None
    if cap > 0:
        capture = (np.zeros((R, cap, C)) if state_update_init is None
                   else np.array(state_update_init, np.float64, copy=True))
    for r in range(R):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        L = t1 - t0
        s = np.zeros((C, K - 1)) if initial_state is None else np.asarray(initial_state[r], np.float64)
        e = np.concatenate([s, x[t0:t1].T], axis=1)                # [C, K - 1 + L]
        for j in range(L):
            z = b + (w * e[:, j:j + K]).sum(axis=1)
            out[t0 + j] = silu(z) if activation == "silu" else z
        final[r] = e[:, L:L + K - 1]
        if cap > 0:
            n = min(L, cap if capture_count is None else max(int(capture_count[r]), 0))
            n = min(n, cap)
            capture[r, :n] = x[t0:t0 + n]
    return out, final, capture


def conv_replay(src_state, state_update, accepted):
    """The committed state advanced by an accepted prefix of captured inputs:
    the last K - 1 of [src, capture[r, 0 .. m - 1]]."""
    src = np.asarray(src_state, np.float64)
    R, C, Km1 = src.shape
    dst = np.zeros_like(src)
    cap = 0 if state_update is None else state_update.shape[1]
    for r in range(R):
        m = min(max(int(accepted[r]), 0), cap)
        e = np.concatenate([src[r], np.asarray(state_update[r, :m], np.float64).T], axis=1) if m else src[r]
        dst[r] = e[:, e.shape[1] - Km1:]
    return dst
