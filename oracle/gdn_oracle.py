"""Plain float64 reference of the GatedDeltaNet (gated delta rule) operator.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the operator library.

What is computed, and where it comes from
-----------------------------------------
The pages describe an operator, com.microsoft::GatedDeltaNet, that runs the
"gated_delta" update rule on packed ragged inputs with an FP32 V-major state
("Add GatedDeltaNet evaluation export for Qwen hybrid models", What changed;
"[CUDA] Add compact GatedDeltaNet operator", Description). They name the rule
and its inputs but do not print it. This oracle takes the published gated
delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving
Mamba2 with Delta Rule", 2024) with the Qwen gate arithmetic computed from the
raw inputs the pages list (raw A_log, dt_bias one scalar per head, a
sigmoid-activated beta; "Export compact GatedDeltaNet state updates for
Qwen3.5/3.8", summary; first page, Dependency):

  x_t     = a_t + dt_bias
  alpha_t = exp(-exp(A_log) * softplus(x_t))          decay, in (0, 1]
  beta_t  = sigmoid(b_t)                               write strength
  k^_t    = k_t / sqrt(|k_t|^2 + eps)                  unit key
  q^_t    = q_t / sqrt(|q_t|^2 + eps) * scale          scale = Dk^-1/2
  u_t     = beta_t * (v_t - alpha_t * S_{t-1} k^_t)    delta (Dv)
  S_t     = alpha_t * S_{t-1} + u_t k^_t^T             state (Dv x Dk)
  o_t     = S_t q^_t

S is stored V-major, one [Dv, Dk] matrix per (request, value head). Value head
h reads key head floor(h / (Hv / Hk)) (grouped keys, "fused linear attention
with GQA" in the first page's Copilot review).

The compact state update ("[CUDA] Add compact GatedDeltaNet operator",
Description: an FP32 capsule packing decay, shared key and delta) holds, per
captured token, alpha for every value head, k^ for every key head and u for
every value head, so that S_t = alpha_t S_{t-1} + u_t k^_t^T can be replayed
from the committed state ("Replay compact fixed state for hybrid decoding",
Summary).

Update rules. The first page names the gated_delta rule and says the exporter
selects among update rules and the operator validates the selection (What
changed; Dependency), without listing the others. They are read here as the
family that the name composes, the same family the Gated DeltaNet paper lays
side by side when it compares linear-attention update rules: the decay gate
alpha and the delta correction each switched on or off.

  gated_delta  S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k^_t) k^_t^T
  delta        the same with alpha_t = 1           (DeltaNet)
  gated        S_t = alpha_t S_{t-1} + v_t k^_t^T   (gated linear attention)
  linear       S_t = S_{t-1} + v_t k^_t^T           (linear attention)

In all four, o_t = S_t q^_t and S_t = alpha_t S_{t-1} + u_t k^_t^T, with u_t the
delta of the delta rules and u_t = v_t for the other two (alpha_t = 1 for the
ungated ones), so the capsule and its replay hold for every rule. The ungated
rules read no decay input (a, A_log, dt_bias), the rules without the delta
correction no beta input (b).

Everything is float64 on the exact values of the (possibly float16-rounded)
inputs. Loops run over tokens; independent heads are batched with numpy.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

L2NORM_EPS = 1e-6


# --------------------------------------------------------------------------
# gates and normalisation
# --------------------------------------------------------------------------
def softplus(x):
    """log(1 + e^x), evaluated in the overflow-free form max(x,0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def log_decay(a, A_log, dt_bias):
    """log alpha = -exp(A_log) * softplus(a + dt_bias); a is [..., Hv]."""
    a = np.asarray(a, dtype=np.float64)
    return -np.exp(np.asarray(A_log, np.float64)) * softplus(a + np.asarray(dt_bias, np.float64))


def gates(a, b, A_log, dt_bias, activation="raw"):
    """(alpha, beta), both float64 [..., Hv].

    "raw": fused native gate arithmetic from raw A_log and per-head dt_bias
    ("[CUDA] Add compact GatedDeltaNet operator", Description).
    "none": precomputed effective gates passed with activation none ("Add
    GatedDeltaNet evaluation export for Qwen hybrid models", What changed):
    alpha = a, beta = b. alpha is clamped to [0, 1], the range of the raw form
    (a reading: the pages only say the gates arrive precomputed).
    """
    if activation == "none":
        return (np.clip(np.asarray(a, np.float64), 0.0, 1.0), np.array(b, np.float64, copy=True))
    if activation != "raw":
        raise ValueError(f"gate activation {activation!r}")
    alpha = np.exp(log_decay(a, A_log, dt_bias))
    beta = 1.0 / (1.0 + np.exp(-np.asarray(b, dtype=np.float64)))
    return alpha, beta


UPDATE_RULES = ("gated_delta", "delta", "gated", "linear")


def rule_parts(rule):
    """(gated, delta) of an update rule: whether it applies the decay alpha, and
    whether it writes the delta beta (v - alpha S k^) rather than v itself."""
    if rule not in UPDATE_RULES:
        raise ValueError(f"update rule {rule!r}")
    return rule in ("gated_delta", "gated"), rule in ("gated_delta", "delta")


def rule_gates(a, b, A_log, dt_bias, activation, rule, num_tokens, Hv):
    """(alpha, beta) [N, Hv] as the rule uses them: alpha = 1 for the ungated
    rules and beta = None for the rules without the delta correction; inputs a
    rule does not read may be None."""
    gated, delta = rule_parts(rule)
    alpha = beta = None
    if gated or delta:
        a_in = a if gated else np.zeros((num_tokens, Hv))
        b_in = b if delta else np.zeros((num_tokens, Hv))
        zeros = np.zeros(Hv)
        alpha, beta = gates(a_in, b_in, A_log if gated else zeros, dt_bias if gated else zeros, activation)
    if not gated:
        alpha = np.ones((num_tokens, Hv))
    if not delta:
        beta = None
    return alpha, beta


def dense_cu_seqlens(num_tokens: int, num_reqs: int) -> np.ndarray:
    """Sequence offsets of the dense rank-4 layout [R, S, ...]: R requests of
    S = N / R tokens each ("[CUDA] Add compact GatedDeltaNet operator",
    Description: ragged and rank-4 inputs)."""
    if num_reqs <= 0 or num_tokens % num_reqs:
        raise ValueError("the dense layout needs N divisible by R")
    return np.arange(num_reqs + 1, dtype=np.int64) * (num_tokens // num_reqs)


def l2normalize(x, eps=L2NORM_EPS):
    """x / sqrt(sum(x^2) + eps) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def key_head_index(Hk: int, Hv: int) -> np.ndarray:
    """Key head read by each value head: h -> floor(h / (Hv / Hk))."""
    if Hk <= 0 or Hv % Hk != 0:
        raise ValueError("Hk must divide Hv")
    return np.arange(Hv) // (Hv // Hk)


def _unit_qk(q, k, Hv, scale):
    """Normalised q^ and k^ of one packed range, expanded to value heads."""
    Dk = q.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    g = key_head_index(q.shape[1], Hv)
    qh = l2normalize(q)[:, g, :] * scale
    kh = l2normalize(k)[:, g, :]
    return qh, kh


# --------------------------------------------------------------------------
# capsule layout
# --------------------------------------------------------------------------
def capsule_width(Hk: int, Hv: int, Dk: int, Dv: int) -> int:
    """Floats per captured token: Hv decays, Hk*Dk unit keys, Hv*Dv deltas."""
    return Hv + Hk * Dk + Hv * Dv


def capsule_sections(Hk: int, Hv: int, Dk: int, Dv: int):
    """Slices of (decay [Hv], shared key [Hk, Dk], delta [Hv, Dv]) in one capsule row.

    Order decay, shared key, delta as the operator description lists them
    ("[CUDA] Add compact GatedDeltaNet operator", Description); no padding.
    """
    s_alpha = slice(0, Hv)
    s_key = slice(Hv, Hv + Hk * Dk)
    s_delta = slice(Hv + Hk * Dk, Hv + Hk * Dk + Hv * Dv)
    return s_alpha, s_key, s_delta


# --------------------------------------------------------------------------
# the token recurrence (the definition)
# --------------------------------------------------------------------------
def recurrence(qh, kh, v, alpha, beta, S0):
    """Run the gated delta rule over one sequence, all heads at once.

    qh, kh : [T, H, Dk] normalised (q^ already scaled)
    v      : [T, H, Dv]
    alpha, beta : [T, H]
    S0     : [H, Dv, Dk]
    Returns (o [T, H, Dv], S_T [H, Dv, Dk], u [T, H, Dv]).
    """
    T, H, Dv = v.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, H, Dv))
    u_all = np.zeros((T, H, Dv))
    for t in range(T):
        a_t = alpha[t][:, None]                                  # [H, 1]
        Sk = np.einsum("hvk,hk->hv", S, kh[t])                   # S_{t-1} k^_t
        u = beta[t][:, None] * (v[t] - a_t * Sk)                 # delta
        S = a_t[:, :, None] * S + u[:, :, None] * kh[t][:, None, :]
        o[t] = np.einsum("hvk,hk->hv", S, qh[t])                 # S_t q^_t
        u_all[t] = u
    return o, S, u_all


def plain_write_recurrence(qh, kh, v, alpha, S0):
    """The rules without the delta correction (gated, and linear with alpha = 1):
    S_t = alpha_t S_{t-1} + v_t k^_t^T, o_t = S_t q^_t; shapes as recurrence.
    Returns (o, S_T, u) with u = v, the capsule's delta for these rules."""
    T, H, Dv = v.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, H, Dv))
    for t in range(T):
        S = alpha[t][:, None, None] * S + v[t][:, :, None] * kh[t][:, None, :]
        o[t] = np.einsum("hvk,hk->hv", S, qh[t])
    return o, S, np.array(v, dtype=np.float64, copy=True)


def gdn_forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, initial_state=None,
                scale=None, state_update_capacity=0, capture_count=None,
                state_update_init=None, gate_activation="raw", num_reqs=None,
                update_rule="gated_delta"):
    """Packed ragged forward by the token recurrence.

    Inputs as the operator takes them (q, k [N, Hk, Dk]; v [N, Hv, Dv]; a, b
    [N, Hv]; A_log, dt_bias [Hv]; cu_seqlens [R + 1], or None with num_reqs for
    the dense layout; initial_state [R, Hv, Dv, Dk] or None for zeros). a and b
    are raw gate inputs or, with gate_activation "none", alpha and beta.
    update_rule is one of UPDATE_RULES. Returns (output [N, Hv, Dv],
    final_state [R, Hv, Dv, Dk], state_update [R, capacity, W] or None).

    With a capacity, request r captures its leading
    n_r = min(len_r, c_r) tokens, c_r being capture_count[r] clamped to
    [0, capacity], or capacity when no counts are given; capsule rows from n_r
    on keep the values of state_update_init (zeros by default). The clamp
    follows the compact capture contract of the causal convolution commit
    embedded in "[CUDA] Add compact GatedDeltaNet operator" (Description: an
    optional per-request capture_count within a bounded capacity; Validation:
    capture-count requirements and capacity bounds), read the same way for the
    GatedDeltaNet capsule.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    cu = (dense_cu_seqlens(q.shape[0], num_reqs) if cu_seqlens is None
          else np.asarray(cu_seqlens, np.int64))
    N, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    R = cu.shape[0] - 1
    _, delta = rule_parts(update_rule)
    alpha, beta = rule_gates(a, b, A_log, dt_bias, gate_activation, update_rule, N, Hv)
    out = np.zeros((N, Hv, Dv))
    final = np.zeros((R, Hv, Dv, Dk))
    cap = int(state_update_capacity)
    capsule = None
    if cap > 0:
        W = capsule_width(Hk, Hv, Dk, Dv)
        capsule = (np.zeros((R, cap, W)) if state_update_init is None
                   else np.array(state_update_init, np.float64, copy=True))
        s_alpha, s_key, s_delta = capsule_sections(Hk, Hv, Dk, Dv)
    for r in range(R):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        S0 = (np.zeros((Hv, Dv, Dk)) if initial_state is None
              else np.asarray(initial_state[r], np.float64))
        if t1 == t0:
            final[r] = S0
            continue
        qh, kh = _unit_qk(q[t0:t1], k[t0:t1], Hv, scale)
        if delta:
            o, S, u = recurrence(qh, kh, v[t0:t1], alpha[t0:t1], beta[t0:t1], S0)
        else:
            o, S, u = plain_write_recurrence(qh, kh, v[t0:t1], alpha[t0:t1], S0)
        out[t0:t1] = o
        final[r] = S
        if cap > 0:
            c_r = cap if capture_count is None else min(max(int(capture_count[r]), 0), cap)
            n = min(t1 - t0, c_r)
            unit_k = l2normalize(k[t0:t0 + n])                   # [n, Hk, Dk]
            for j in range(n):
                capsule[r, j, s_alpha] = alpha[t0 + j]
                capsule[r, j, s_key] = unit_k[j].reshape(-1)
                capsule[r, j, s_delta] = u[j].reshape(-1)
    return out, final, capsule


def gdn_replay(src_state, state_update, accepted, Hk, Hv, Dk, Dv):
    """Advance the committed state by an accepted capsule prefix.

    dst[r, h] = src[r, h]; then for j < m_r:
    dst[r, h] <- alpha_j[h] * dst[r, h] + u_j[h] k^_j[g(h)]^T.
    ("Replay compact fixed state for hybrid decoding", Summary: replay only an
    accepted prefix into an inactive state bank.) m_r is accepted[r] clamped
    to [0, capacity], capacity being the number of capsule rows: a replay never
    reads past the rows a request owns (the capacity bound of the compact
    capture contract in "[CUDA] Add compact GatedDeltaNet operator", embedded
    causal convolution commit, Validation).
    """
    src = np.asarray(src_state, np.float64)
    cap_rows = np.asarray(state_update, np.float64)
    R = src.shape[0]
    capacity = cap_rows.shape[1]
    s_alpha, s_key, s_delta = capsule_sections(Hk, Hv, Dk, Dv)
    g = key_head_index(Hk, Hv)
    dst = np.array(src, copy=True)
    for r in range(R):
        m = min(max(int(accepted[r]), 0), capacity)
        for j in range(m):
            row = cap_rows[r, j]
            al = row[s_alpha]                                   # [Hv]
            kk = row[s_key].reshape(Hk, Dk)[g]                  # [Hv, Dk]
            uu = row[s_delta].reshape(Hv, Dv)                   # [Hv, Dv]
            dst[r] = al[:, None, None] * dst[r] + uu[:, :, None] * kk[:, None, :]
    return dst


# --------------------------------------------------------------------------
# chunked (WY / UT) form: an exact algebraic rewrite of the recurrence
# --------------------------------------------------------------------------
def chunk_step(qh, kh, v, log_alpha, beta, S0):
    """One chunk of L tokens, every head, in the chunkwise-parallel form.

    With g_r = sum_{i<=r} log alpha_i (reset at the chunk start) and
    A[r, i] = beta_r exp(g_r - g_i) (k^_r . k^_i) for i < r:
      U   solves (I + A) U = diag(beta) (V - diag(e^g) K^ S0^T)
      O   = diag(e^g) Q^ S0^T + (M o Q^ K^^T) U,  M[r, i] = exp(g_r - g_i), i <= r
      S_L = e^{g_L} S0 + U^T diag(e^{g_L - g}) K^
    The rows of U are the per-token deltas u_t of the recurrence.
    (The UT/WY chunk form of DeltaNet and Gated DeltaNet: Yang et al. 2024,
    "Parallelizing Linear Transformers with the Delta Rule over Sequence
    Length", and the Gated DeltaNet paper.)
    """
    L, H, Dk = kh.shape
    Dv = v.shape[2]
    o = np.zeros((L, H, Dv))
    S_out = np.zeros((H, Dv, Dk))
    g = np.cumsum(log_alpha, axis=0)                             # [L, H]
    strict = np.tril(np.ones((L, L), dtype=bool), -1)
    incl = np.tril(np.ones((L, L), dtype=bool), 0)
    eye = np.eye(L)
    for h in range(H):
        K, Q, V, gh, bh = kh[:, h], qh[:, h], v[:, h], g[:, h], beta[:, h]
        diff = gh[:, None] - gh[None, :]                         # g_r - g_i
        A = np.where(strict, bh[:, None] * np.exp(np.where(strict, diff, -np.inf)) * (K @ K.T), 0.0)
        rhs = bh[:, None] * (V - np.exp(gh)[:, None] * (K @ S0[h].T))
        U = solve_triangular(eye + A, rhs, lower=True, unit_diagonal=True)
        M = np.exp(np.where(incl, diff, -np.inf))
        o[:, h] = np.exp(gh)[:, None] * (Q @ S0[h].T) + (M * (Q @ K.T)) @ U
        S_out[h] = np.exp(gh[-1]) * S0[h] + U.T @ (np.exp(gh[-1] - gh)[:, None] * K)
    return o, S_out


def chunk_step_plain_write(qh, kh, v, log_alpha, S0):
    """One chunk of the rules without the delta correction: the deltas are the
    values themselves (U = V), so
      O   = diag(e^g) Q^ S0^T + (M o Q^ K^^T) V
      S_L = e^{g_L} S0 + V^T diag(e^{g_L - g}) K^."""
    L, H, Dk = kh.shape
    Dv = v.shape[2]
    o = np.zeros((L, H, Dv))
    S_out = np.zeros((H, Dv, Dk))
    g = np.cumsum(log_alpha, axis=0)
    incl = np.tril(np.ones((L, L), dtype=bool), 0)
    for h in range(H):
        K, Q, V, gh = kh[:, h], qh[:, h], v[:, h], g[:, h]
        M = np.exp(np.where(incl, gh[:, None] - gh[None, :], -np.inf))
        o[:, h] = np.exp(gh)[:, None] * (Q @ S0[h].T) + (M * (Q @ K.T)) @ V
        S_out[h] = np.exp(gh[-1]) * S0[h] + V.T @ (np.exp(gh[-1] - gh)[:, None] * K)
    return o, S_out


def chunked_forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, initial_state=None,
                    scale=None, chunk=64, update_rule="gated_delta"):
    """Packed ragged forward in the chunked form; chunks start at each sequence start."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    R = cu.shape[0] - 1
    gated, delta = rule_parts(update_rule)
    la = log_decay(a, A_log, dt_bias) if gated else np.zeros((N, Hv))
    beta = 1.0 / (1.0 + np.exp(-np.asarray(b, np.float64))) if delta else None
    out = np.zeros((N, Hv, Dv))
    final = np.zeros((R, Hv, Dv, Dk))
    for r in range(R):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        S = (np.zeros((Hv, Dv, Dk)) if initial_state is None
             else np.array(initial_state[r], np.float64, copy=True))
        for c0 in range(t0, t1, chunk):
            c1 = min(c0 + chunk, t1)
            qh, kh = _unit_qk(q[c0:c1], k[c0:c1], Hv, scale)
            if delta:
                o, S = chunk_step(qh, kh, v[c0:c1], la[c0:c1], beta[c0:c1], S)
            else:
                o, S = chunk_step_plain_write(qh, kh, v[c0:c1], la[c0:c1], S)
            out[c0:c1] = o
        final[r] = S
    return out, final
