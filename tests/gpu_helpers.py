"""Shared helpers of the GPU tests: device copies of seeded inputs, one call of
the library through its binding, and the tolerance measures."""
from __future__ import annotations

import numpy as np

TOL_F32_REL = 1e-4          # FP32 I/O: max|x - y| / max|y|
TOL_F16_OUT_ABS = 2e-2      # FP16 I/O: output max-abs error
TOL_F16_STATE_RL2 = 1e-3    # FP16 I/O: final-state relative L2 error
TOL_REPLAY_REL = 1e-5       # replay vs the GPU's own recurrence: max|x - y| / max|y|


def rel_max(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = float(np.max(np.abs(y))) if y.size else 0.0
    return float(np.max(np.abs(x - y))) / den if den > 0 else float(np.max(np.abs(x - y), initial=0.0))


def rel_l2(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = float(np.linalg.norm(y))
    return float(np.linalg.norm(x - y)) / den if den > 0 else float(np.linalg.norm(x - y))


def max_abs(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.max(np.abs(x - y), initial=0.0))


def dev(x, torch, dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def device_inputs(inp, torch):
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    d["initial_state"] = dev(inp["initial_state"], torch)
    return d


RULE_NAMES = ("gated_delta", "delta", "gated", "linear")     # gdn_rule codes 0 .. 3


def rule_reads(rule):
    """(reads the decay input a, reads beta b) of an update rule name."""
    return rule in ("gated_delta", "gated"), rule in ("gated_delta", "delta")


def run_forward(inp, torch, gdn, *, in_place=False, write_final=True, capacity=0,
                capture_count=None, poison=None, plan=None, host_cu=True, workspace=True,
                scale=0.0, gate="raw", dense=False, rule="gated_delta"):
    """One gdn_forward call on fresh device copies; returns numpy results.

    gate "none": a, b are passed as effective gates without A_log, dt_bias.
    dense: no cu_seqlens (every request holds N / R tokens).
    rule: update rule name; inputs the rule does not read are passed as NULL."""
    d = device_inputs(inp, torch)
    if gate == "none":
        d["A_log"] = d["dt_bias"] = None
    reads_a, reads_b = rule_reads(rule)
    if not reads_a:
        d["a"] = d["A_log"] = d["dt_bias"] = None
    if not reads_b:
        d["b"] = None
    N, Hv, Dv = inp["v"].shape
    R = len(inp["cu_seqlens"]) - 1
    Hk, Dk = inp["Hk"], inp["Dk"]
    out = torch.full((N, Hv, Dv), float("nan"), dtype=d["v"].dtype, device="cuda")
    init = d["initial_state"]
    fin = None
    if write_final:
        if in_place:
            if init is None:
                raise ValueError("in place needs an initial state")
            fin = init
        else:
            fin = torch.full((R, Hv, Dv, Dk), float("nan"), dtype=torch.float32, device="cuda")
    su = None
    if capacity > 0:
        W = gdn.capsule_width(Hk, Hv, Dk, Dv)
        su = torch.full((R, capacity, W), np.float32(poison if poison is not None else np.nan),
                        dtype=torch.float32, device="cuda")
    cc = dev(capture_count, torch) if capture_count is not None else None
    plan_code = gdn.PLAN_AUTO if plan is None else plan
    cu_host = inp["cu_seqlens"] if host_cu and not dense else None
    ws = None
    if workspace:
        nbytes = gdn.gdn_forward_workspace_bytes(N, R, Hk, Hv, Dk, Dv,
                                                 gdn.GDN_F16 if inp["io_dtype"] == "f16" else gdn.GDN_F32,
                                                 capacity=capacity, plan=plan_code,
                                                 cu_seqlens_host=cu_host)
        if nbytes:
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                    None if dense else d["cu_seqlens"], out, initial_state=init, final_state=fin,
                    state_update=su, capture_count=cc, cu_seqlens_host=cu_host,
                    state_update_capacity=capacity, plan=plan_code, workspace=ws, scale=scale,
                    gate_activation=gdn.GATE_NONE if gate == "none" else gdn.GATE_RAW,
                    num_reqs=R if dense else None, update_rule=RULE_NAMES.index(rule))
    torch.cuda.synchronize()
    res = {"output": out.float().cpu().numpy(),
           "final_state": None if fin is None else fin.cpu().numpy(),
           "state_update": None if su is None else su.cpu().numpy(),
           "initial_after": None if init is None else init.cpu().numpy()}
    return res


def oracle_forward(inp, O, capacity=0, capture_count=None, poison=None, scale=None, gate="raw",
                   rule="gated_delta"):
    init = None
    if capacity > 0:
        W = O.capsule_width(inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"])
        init = np.full((len(inp["cu_seqlens"]) - 1, capacity, W),
                       np.nan if poison is None else poison)
    return O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                         inp["dt_bias"], inp["cu_seqlens"], inp["initial_state"],
                         scale=scale, state_update_capacity=capacity,
                         capture_count=capture_count, state_update_init=init,
                         gate_activation=gate, update_rule=rule)


def sample_heads_inputs(inp, heads):
    """The sub-problem of the given value heads only, with each head's key head
    repeated (grouped keys equal repeat-interleaved keys; pinned by the oracle's
    GQA check), so the oracle can run full-length sequences on a few heads."""
    heads = np.asarray(heads)
    G = inp["Hv"] // inp["Hk"]
    kh = heads // G
    sub = dict(inp)
    sub["q"] = inp["q"][:, kh]
    sub["k"] = inp["k"][:, kh]
    sub["v"] = inp["v"][:, heads]
    sub["a"] = np.ascontiguousarray(inp["a"][:, heads])
    sub["b"] = np.ascontiguousarray(inp["b"][:, heads])
    sub["A_log"] = inp["A_log"][heads]
    sub["dt_bias"] = inp["dt_bias"][heads]
    if inp["initial_state"] is not None:
        sub["initial_state"] = inp["initial_state"][:, heads]
    sub["Hk"] = sub["Hv"] = len(heads)
    return sub


def _oracle_heads_task(sub):
    """Worker of oracle_forward_all_heads: the float64 recurrence on one head group."""
    from oracle import gdn_oracle as O
    out, fin, _ = O.gdn_forward(sub["q"], sub["k"], sub["v"], sub["a"], sub["b"], sub["A_log"],
                                sub["dt_bias"], sub["cu_seqlens"], sub["initial_state"])
    return out, fin


def oracle_forward_all_heads(inp, heads_per_task=4, workers=None):
    """The float64 recurrence over every value head of a large workload, split into
    groups of heads (sample_heads_inputs) that run in parallel worker processes.
    The workers are started fresh (spawn) and compute on the CPU only. Returns
    (output [N, Hv, Dv], final_state [R, Hv, Dv, Dk]) assembled in head order."""
    import multiprocessing as mp
    import os
    from concurrent.futures import ProcessPoolExecutor

    Hv = inp["Hv"]
    groups = [list(range(h, min(h + heads_per_task, Hv))) for h in range(0, Hv, heads_per_task)]
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(groups)))
    subs = [sample_heads_inputs(inp, hs) for hs in groups]
    N, _, Dv = inp["v"].shape
    R = len(inp["cu_seqlens"]) - 1
    Dk = inp["q"].shape[2]
    out = np.zeros((N, Hv, Dv))
    fin = np.zeros((R, Hv, Dv, Dk))
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        for hs, (o, f) in zip(groups, ex.map(_oracle_heads_task, subs)):
            out[:, hs] = o
            fin[:, hs] = f
    return out, fin


def assert_parity(io_dtype, out, ref_out, fin=None, ref_fin=None, what=""):
    if io_dtype == "f32":
        e_o = rel_max(out, ref_out)
        assert e_o <= TOL_F32_REL, f"{what} output rel-max {e_o:.3e}"
        if fin is not None:
            e_s = rel_max(fin, ref_fin)
            assert e_s <= TOL_F32_REL, f"{what} final-state rel-max {e_s:.3e}"
    else:
        e_o = max_abs(out, ref_out)
        assert e_o <= TOL_F16_OUT_ABS, f"{what} output max-abs {e_o:.3e}"
        if fin is not None:
            e_s = rel_l2(fin, ref_fin)
            assert e_s <= TOL_F16_STATE_RL2, f"{what} final-state rel-L2 {e_s:.3e}"


def effective_gate_inputs(inp, seed):
    """The inputs with a, b replaced by effective gates (activation none): alpha
    mostly in [0.5, 1), with exact 1s, exact 0s (a state reset) and values past
    either end of [0, 1] (clamped by the operator and the oracle alike), and
    beta in [0, 1)."""
    rng = np.random.default_rng(seed)
    e = dict(inp)
    alpha = rng.uniform(0.5, 1.0, inp["a"].shape)
    alpha.flat[::7] = 1.0
    alpha.flat[3::11] = 0.0
    alpha.flat[5::13] = 1.3
    alpha.flat[6::17] = -0.2
    e["a"] = alpha.astype(np.float32)
    e["b"] = rng.uniform(0.0, 1.0, inp["b"].shape).astype(np.float32)
    return e
