"""The float64 oracle timed on the host's cores: the CPU baseline printed beside
the GPU figures by bench.py.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: it times the oracle as it
stands (oracle.gdn_oracle, unchanged) and computes nothing of the method itself.
The workload's value heads are split into groups (grouped keys expanded per
value head, which the oracle's GQA pin shows to be the same computation); one
single-threaded worker process per group runs the oracle for a bounded time.
"""
from __future__ import annotations

import os
import time

import numpy as np


def _head_groups(Hv, workers):
    per = -(-Hv // workers)
    return [list(range(h, min(h + per, Hv))) for h in range(0, Hv, per)]


def _sub_heads(inp, heads, n_tokens=None):
    """Inputs of the given value heads only, each with its key head (grouped keys
    equal repeat-interleaved keys), optionally cut to the first n_tokens tokens."""
    heads = np.asarray(heads)
    G = inp["Hv"] // inp["Hk"]
    kh = heads // G
    T = inp["q"].shape[0] if n_tokens is None else n_tokens
    sub = {"q": np.ascontiguousarray(inp["q"][:T, kh]), "k": np.ascontiguousarray(inp["k"][:T, kh]),
           "v": np.ascontiguousarray(inp["v"][:T, heads]), "a": np.ascontiguousarray(inp["a"][:T, heads]),
           "b": np.ascontiguousarray(inp["b"][:T, heads]), "A_log": inp["A_log"][heads],
           "dt_bias": inp["dt_bias"][heads], "cu_seqlens": inp["cu_seqlens"],
           "initial_state": None if inp["initial_state"] is None else inp["initial_state"][:, heads]}
    if inp.get("capacity"):
        sub["capacity"] = inp["capacity"]
        sub["accepted"] = inp["accepted"]
    return sub


def _oracle_worker(task):
    """One CPU worker of the oracle baseline: the float64 oracle, unchanged, on one
    group of value heads, one thread, for about `seconds`. Returns (tokens, seconds)."""
    kind, sub, seconds = task
    from threadpoolctl import threadpool_limits
    from oracle import gdn_oracle as O
    N = sub["q"].shape[0]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        tokens = 0
        if kind == "decode":
            state = sub["initial_state"]
            while True:
                _, state, _ = O.gdn_forward(sub["q"], sub["k"], sub["v"], sub["a"], sub["b"], sub["A_log"],
                                            sub["dt_bias"], sub["cu_seqlens"], state)
                tokens += N
                if time.perf_counter() - t0 >= seconds:
                    break
        elif kind == "verify_replay":
            Hk = Hv = sub["v"].shape[1]
            Dk, Dv = sub["q"].shape[2], sub["v"].shape[2]
            while True:
                _, _, capsule = O.gdn_forward(sub["q"], sub["k"], sub["v"], sub["a"], sub["b"], sub["A_log"],
                                              sub["dt_bias"], sub["cu_seqlens"], sub["initial_state"],
                                              state_update_capacity=sub["capacity"])
                O.gdn_replay(sub["initial_state"], capsule, sub["accepted"], Hk, Hv, Dk, Dv)
                tokens += N
                if time.perf_counter() - t0 >= seconds:
                    break
        else:
            # prefill: the requests in order, each in blocks of at most 256 tokens that
            # carry the request's state, until the time is up or the sample ends
            cu = sub["cu_seqlens"]
            done = False
            for r in range(len(cu) - 1):
                state = sub["initial_state"][r:r + 1]
                for b0 in range(int(cu[r]), int(cu[r + 1]), 256):
                    b1 = min(b0 + 256, int(cu[r + 1]), N)
                    if b1 <= b0:
                        break
                    _, state, _ = O.gdn_forward(sub["q"][b0:b1], sub["k"][b0:b1], sub["v"][b0:b1],
                                                sub["a"][b0:b1], sub["b"][b0:b1], sub["A_log"], sub["dt_bias"],
                                                np.array([0, b1 - b0]), state)
                    tokens += b1 - b0
                    if time.perf_counter() - t0 >= seconds:
                        done = True
                        break
                if done or int(cu[r + 1]) >= N:
                    break
        return tokens, time.perf_counter() - t0


def cpu_baseline(inp, kind, seconds, max_tokens=None):
    """The float64 oracle as it stands, timed on this host's cores: the workload's
    value heads split into groups, one single-threaded worker process per group
    (at most 16, the host's CPU share), all running together for about `seconds`.
    The rate is that of the slowest group (every head of a token must be done).
    kind: "decode" (consecutive steps, the state threaded through), "verify_replay"
    (verify with capsule, then replay of the accepted prefix, per step) or
    "prefill" (the packed tokens in order, the token recurrence, up to max_tokens)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    Hv = inp["Hv"]
    avail = len(os.sched_getaffinity(0))
    workers = max(1, min(16, avail, Hv))
    groups = _head_groups(Hv, workers)
    subs = [_sub_heads(inp, hs, max_tokens) for hs in groups]
    with ProcessPoolExecutor(max_workers=len(groups), mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_worker, [(kind, sub, seconds) for sub in subs]))
    rate = min(t / el for t, el in res)
    tokens = min(t for t, _ in res)
    el = max(el for _, el in res)
    what = {"decode": "consecutive decode steps (the state threaded through)",
            "verify_replay": "verify steps with capsule capture, each followed by the replay of the accepted prefix",
            "prefill": "the packed tokens in order, blocks of at most 256 tokens carrying each request's state"}[kind]
    return {"value": rate, "unit": "tokens/s", "cores": len(groups), "kind": "oracle",
            "sample": f"{what}: {tokens} tokens of every one of the {Hv} value heads in {el:.1f} s; "
                      f"numpy float64 token recurrence, {len(groups)} single-threaded worker processes "
                      f"of {len(groups[0])} heads each; host: {os.cpu_count()} logical CPUs, "
                      f"{avail} available to this process"}
