"""Benchmark of the GatedDeltaNet operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the operator's hot path over one batch of synthetic
input. The default workload is the batched decode step (64 requests x 1 token,
Hk=16, Hv=32, Dk=Dv=128, fp16 I/O, FP32 V-major state updated in place), whose
time is dominated by gdn_decode streaming the 128 MiB state through HBM. To
keep the state out of the 256 MB Infinity Cache, consecutive steps rotate over
several state banks (>= 512 MiB in total), so every step reads cold state.

Prints one JSON line: tokens/s, ms per step, the dominant kernel's roofline
(algorithmic bytes / its average duration from HIP events on the launch
stream, against the 8 TB/s HBM peak) and the float64 oracle timed on this
host's cores on a bounded sample of the same workload. The line also carries,
under "workloads", the same measurements for the operator's other workloads:
speculative verify + replay (HBM roofline), the ragged and long prefills
(fp16 MFMA roofline), the decode step with precomputed effective gates in the
dense rank-4 layout, the compact causal convolution upstream of the operator
on a prefill and a decode batch (HBM roofline), and the speculative step over a
fixed-state pool (verify, replay, publish), and the decode step with a K-major
state; --workload NAME times just one of them.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "GDN tokens/s + achieved HBM GB/s (decode/replay), MFMA % (prefill)"
BANK_TARGET_BYTES = 512 * 2 ** 20

# HBM traffic per launch (per step for workloads of several kernels), from rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE runs of that workload (KiB per dispatch, summed over
# the step's kernels), each scaled by what the same counter reads for the 128 MiB
# hbm_copy workload (FETCH_SIZE reads 65547.7 KiB for 131072 KiB copied: factor
# 1.9996; WRITE_SIZE is exact: factor 1.0000). Keyed by the hash of the kernels'
# sources: a changed kernel reports null until its counters are taken again.
MEASURED_TRAFFIC = {
    "batched_decode": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "90c96b595bdee1ba", "fetch_kib": 66933.0, "write_kib": 131598.7,
        "bytes": 271811346},
    "decode_effective_dense": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "90c96b595bdee1ba", "fetch_kib": 66928.6, "write_kib": 131592.9,
        "bytes": 271796440},
    "decode_kmajor": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_kmajor.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "5002d5fb8d5d6360", "fetch_kib": 66936.1, "write_kib": 131593.5,
        "bytes": 271812403},
    "spec_verify_replay": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_replay.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "9d6f7262a47c98f6", "fetch_kib": 51133.3, "write_kib": 52119.2,
        "bytes": 158072430},
    "spec_step_fused": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "90c96b595bdee1ba", "fetch_kib": 26530.9, "write_kib": 52096.4,
        "bytes": 107672220},
    "spec_step_pooled": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_replay.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "9d6f7262a47c98f6", "fetch_kib": 51135.8, "write_kib": 52119.9,
        "bytes": 158078237},
    "spec_step_pooled_fused": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_replay.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "9d6f7262a47c98f6", "fetch_kib": 26532.9, "write_kib": 52092.6,
        "bytes": 107672440},
    "ragged_prefill": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_chunk.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "8a28ff8159b58b10", "fetch_kib": 258792.7, "write_kib": 240761.7,
        "bytes": 776452826},
    "long_prefill": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_chunk.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "8a28ff8159b58b10", "fetch_kib": 669508.5, "write_kib": 715781.8,
        "bytes": 2103869140},
    "conv_prefill": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_conv.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "8efa3ae12fc932a2", "fetch_kib": 124275.1, "write_kib": 246403.3,
        "bytes": 506786802},
    "conv_decode": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_conv.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "8efa3ae12fc932a2", "fetch_kib": 3712.1, "write_kib": 7168.0,
        "bytes": 14941110},
    "conv_decode_fused": {"sources": ['gateddeltanet_recurrence_amd/csrc/gdn_recurrent.hip', 'gateddeltanet_recurrence_amd/csrc/gdn_common.h', 'gateddeltanet_recurrence_amd/csrc/gdn_kernels.h'],
        "sha256_16": "90c96b595bdee1ba", "fetch_kib": 69403.1, "write_kib": 137757.6,
        "bytes": 283176033},
}


def measured_traffic(kernel):
    """Calibrated HBM bytes per launch of `kernel`, or None if its sources changed."""
    import hashlib
    rec = MEASURED_TRAFFIC.get(kernel)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes"] if h.hexdigest()[:16] == rec["sha256_16"] else None


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _dev(x, torch):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


# --------------------------------------------------------------------- decode
def decode_bytes(inp) -> int:
    """Algorithmic HBM bytes of one decode launch: the state read and written once,
    q, k, v, output, gates and cu_seqlens read/written once."""
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R = len(inp["cu_seqlens"]) - 1
    io = inp["q"].dtype.itemsize
    return (2 * R * Hv * Dv * Dk * 4 + 2 * N * Hk * Dk * io + 2 * N * Hv * Dv * io
            + 2 * N * Hv * 4 + 2 * Hv * 4 + (R + 1) * 4)


def run_decode(args, torch, gdn):
    from gdn_workloads import workload_inputs
    inp = workload_inputs("batched_decode")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R = len(inp["cu_seqlens"]) - 1
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    state_bytes = R * Hv * Dv * Dk * 4
    n_banks = max(2, -(-BANK_TARGET_BYTES // state_bytes))
    init = _dev(inp["initial_state"], torch)
    banks = [init.clone() for _ in range(n_banks)]
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    host_cu = inp["cu_seqlens"]
    stream = torch.cuda.current_stream()

    def step(i):
        s = banks[i % n_banks]
        gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=s, final_state=s,
                        cu_seqlens_host=host_cu, plan=gdn.PLAN_RECURRENT, stream=stream)

    _log(f"decode: R={R} Hv={Hv} D={Dk} banks={n_banks} warmup={args.warmup} steps={args.steps}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / args.steps
    nbytes = decode_bytes(inp)
    achieved = nbytes / (ms_step * 1e-3) / 1e9
    traffic = measured_traffic("batched_decode")
    # context only: single-call times, and one bank reused every step (its 128 MiB
    # can then stay in the 256 MB Infinity Cache between steps)
    per_call = _per_call(torch, step, 50, args.warmup + args.steps)
    hot_ms = _time_steps(torch, lambda i: step(0), 100, 10)
    hot = {"ms_per_step": hot_ms, "achieved_GBps": nbytes / (hot_ms * 1e-3) / 1e9}
    line = {
        "metric": METRIC, "value": N / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "batched_decode", "requests": R, "tokens_per_step": N,
                   "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv, "io_dtype": "f16",
                   "state": "fp32 V-major [64,32,128,128], in place", "state_banks": n_banks},
        "roofline": {"bound": "hbm", "kernel": "gdn_decode", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "event_us_per_launch": ms_step * 1e3},
        "per_call": per_call,
        "hot_single_bank": hot,
    }
    return line, inp


def run_decode_effective_dense(args, torch, gdn):
    """The batched decode step in the operator's other input forms: precomputed
    effective gates (activation none; alpha in [0.5, 1), beta in [0, 1), synthetic)
    and the dense rank-4 layout [R, 1, H, D] (no cu_seqlens). Same kernel and
    state traffic as the batched decode; A_log, dt_bias and cu_seqlens are not read."""
    import numpy as np
    from gdn_workloads import workload_inputs
    inp = workload_inputs("batched_decode")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R = len(inp["cu_seqlens"]) - 1
    rng = np.random.default_rng(7)
    alpha = torch.from_numpy(rng.uniform(0.5, 1.0, (N, Hv)).astype(np.float32)).cuda()
    beta = torch.from_numpy(rng.uniform(0.0, 1.0, (N, Hv)).astype(np.float32)).cuda()
    q, k, v = (_dev(inp[n], torch).reshape(R, N // R, *inp[n].shape[1:]) for n in ("q", "k", "v"))
    state_bytes = R * Hv * Dv * Dk * 4
    n_banks = max(2, -(-BANK_TARGET_BYTES // state_bytes))
    banks = [_dev(inp["initial_state"], torch) for _ in range(n_banks)]
    out = torch.empty_like(v)
    a4, b4 = alpha.reshape(R, N // R, Hv), beta.reshape(R, N // R, Hv)

    def step(i):
        s = banks[i % n_banks]
        gdn.gdn_forward(q, k, v, a4, b4, None, None, None, out, initial_state=s, final_state=s,
                        gate_activation=gdn.GATE_NONE, plan=gdn.PLAN_RECURRENT)

    _log(f"decode, effective gates, dense layout: R={R} Hv={Hv} banks={n_banks}")
    ms = _time_steps(torch, step, args.steps, args.warmup)
    nbytes = decode_bytes(inp) - 2 * Hv * 4 - (R + 1) * 4
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "config": {"tokens": N, "requests": R, "layout": "dense [R, 1, H, D]",
                       "gates": "effective (activation none)", "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv},
            "roofline": {"bound": "hbm", "kernel": "gdn_decode", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_effective_dense"),
                         "algorithmic_bytes_per_step": nbytes}}


def run_decode_kmajor(args, torch, gdn):
    """The batched decode step with the K-major state layout [R, Hv, Dk, Dv] (the
    dense LinearAttention layout): the gdn_decode_kmajor kernel, same state traffic."""
    from gdn_workloads import workload_inputs
    inp = workload_inputs("batched_decode")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R = len(inp["cu_seqlens"]) - 1
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    state_bytes = R * Hv * Dv * Dk * 4
    n_banks = max(2, -(-BANK_TARGET_BYTES // state_bytes))
    km = np.ascontiguousarray(np.swapaxes(inp["initial_state"], -1, -2))
    banks = [_dev(km, torch) for _ in range(n_banks)]
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    host_cu = inp["cu_seqlens"]

    def step(i):
        s = banks[i % n_banks]
        gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=s, final_state=s,
                        cu_seqlens_host=host_cu, plan=gdn.PLAN_RECURRENT, state_layout=gdn.STATE_K_MAJOR)

    _log(f"decode, K-major state: R={R} Hv={Hv} banks={n_banks}")
    ms = _time_steps(torch, step, args.steps, args.warmup)
    nbytes = decode_bytes(inp)
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "config": {"tokens": N, "requests": R, "state": "fp32 K-major [64,32,128,128], in place",
                       "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv, "state_banks": n_banks},
            "roofline": {"bound": "hbm", "kernel": "gdn_decode_kmajor", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_kmajor"),
                         "algorithmic_bytes_per_step": nbytes}}


def _time_steps(torch, step, steps, warmup, min_warm_s=0.0):
    """Average ms per step of `step(i)` over `steps` calls, HIP events on the launch stream.
    With min_warm_s, the untimed warmup goes on (in batches of `warmup` calls) until it
    has run at least that long: after lighter work the GPU's clocks take tens of
    milliseconds to settle, longer than a few calls of a short workload."""
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    done = 0
    while True:
        for i in range(warmup):
            step(done + i)
        done += warmup
        torch.cuda.synchronize()
        if warmup <= 0 or time.perf_counter() - t0 >= min_warm_s:
            break
    warmup = done
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        step(warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def _per_call(torch, step, calls, start):
    """Distribution of single-call times: `calls` further steps, each bracketed by
    its own HIP events on the launch stream (after the timed region, not part of it)."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for j, (e0, e1) in enumerate(evs):
        e0.record(stream)
        step(start + j)
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    def quantile(f):
        return 1e3 * t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]

    return {"calls": calls, "median_us": quantile(0.5), "p10_us": quantile(0.1), "p90_us": quantile(0.9)}


def run_verify_replay(args, torch, gdn):
    """Speculative verify (capsule, committed bank read-only) then replay of the
    accepted prefix into the inactive bank, per step."""
    from gdn_workloads import workload_inputs
    inp = workload_inputs("spec_verify_replay")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R, cap = len(inp["cu_seqlens"]) - 1, inp["capacity"]
    W = gdn.capsule_width(Hk, Hv, Dk, Dv)
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    acc_host = inp["accepted"]
    acc = _dev(acc_host, torch)
    state_bytes = R * Hv * Dv * Dk * 4
    n_banks = max(4, 2 * -(-(3 * BANK_TARGET_BYTES // 2) // (2 * state_bytes)))
    init = _dev(inp["initial_state"], torch)
    banks = [init.clone() for _ in range(n_banks)]
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    capsule = torch.empty((R, cap, W), dtype=torch.float32, device="cuda")
    host_cu = inp["cu_seqlens"]

    def step(i):
        committed = banks[(2 * i) % n_banks]
        inactive = banks[(2 * i + 1) % n_banks]
        gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=committed,
                        state_update=capsule, state_update_capacity=cap, cu_seqlens_host=host_cu,
                        plan=gdn.PLAN_RECURRENT)
        gdn.gdn_replay(committed, capsule, acc, inactive, num_k_heads=Hk, state_update_capacity=cap,
                       accepted_host=acc_host)

    _log(f"verify+replay: R={R} T=4 Hv={Hv} banks={n_banks}")
    ms = _time_steps(torch, step, args.steps, args.warmup)
    per_call = _per_call(torch, step, 50, args.warmup + args.steps)   # single-call latency
    io = 2
    verify_bytes = (state_bytes + R * cap * W * 4 + 2 * N * Hk * Dk * io + 2 * N * Hv * Dv * io
                    + 2 * N * Hv * 4 + 2 * Hv * 4 + (R + 1) * 4)
    replay_bytes = 2 * state_bytes + int(acc_host.sum()) * W * 4 + R * 4
    nbytes = verify_bytes + replay_bytes
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "per_call": per_call,
            "config": {"requests": R, "draft_tokens": 4, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                       "capacity": cap, "accepted": acc_host.tolist(), "state_banks": n_banks},
            "roofline": {"bound": "hbm", "kernel": "gdn_capsule+gdn_replay", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": measured_traffic("spec_verify_replay"), "algorithmic_bytes_per_step": nbytes,
                         "verify_bytes": verify_bytes, "replay_bytes": replay_bytes}}


def run_spec_step_fused(args, torch, gdn):
    """The speculative step as one gdn_replay_forward call: the previous step's
    accepted prefix replayed from the committed bank into the inactive bank and
    this step's verify from that state, the committed bank read once. The banks
    rotate as in spec_verify_replay; each step replays the capsule the previous
    step wrote (two capsule buffers alternate)."""
    from gdn_workloads import workload_inputs
    inp = workload_inputs("spec_verify_replay")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R, cap = len(inp["cu_seqlens"]) - 1, inp["capacity"]
    W = gdn.capsule_width(Hk, Hv, Dk, Dv)
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    acc_host = inp["accepted"]
    acc = _dev(acc_host, torch)
    state_bytes = R * Hv * Dv * Dk * 4
    n_banks = max(4, 2 * -(-(3 * BANK_TARGET_BYTES // 2) // (2 * state_bytes)))
    init = _dev(inp["initial_state"], torch)
    banks = [init.clone() for _ in range(n_banks)]
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    caps = [torch.empty((R, cap, W), dtype=torch.float32, device="cuda") for _ in range(2)]
    host_cu = inp["cu_seqlens"]
    # a real previous capsule for the first step: one verify from the committed bank
    gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=banks[0], state_update=caps[1],
                    state_update_capacity=cap, cu_seqlens_host=host_cu, plan=gdn.PLAN_RECURRENT)

    def step(i):
        gdn.gdn_replay_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=banks[(2 * i) % n_banks],
                               state_update=caps[i % 2], state_update_capacity=cap, cu_seqlens_host=host_cu,
                               prev_state_update=caps[(i + 1) % 2], accepted=acc, accepted_host=acc_host,
                               replay_state=banks[(2 * i + 1) % n_banks], plan=gdn.PLAN_RECURRENT)

    _log(f"fused replay+verify: R={R} T=4 Hv={Hv} banks={n_banks}")
    ms = _time_steps(torch, step, args.steps, args.warmup)
    per_call = _per_call(torch, step, 50, args.warmup + args.steps)
    io = 2
    nbytes = (2 * state_bytes + int(acc_host.sum()) * W * 4 + R * cap * W * 4 + 2 * N * Hk * Dk * io
              + 2 * N * Hv * Dv * io + 2 * N * Hv * 4 + 2 * Hv * 4 + (R + 1) * 4 + R * 4)
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "per_call": per_call,
            "config": {"requests": R, "draft_tokens": 4, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                       "capacity": cap, "accepted": acc_host.tolist(), "state_banks": n_banks},
            "roofline": {"bound": "hbm", "kernel": "gdn_replay_verify", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": measured_traffic("spec_step_fused"), "algorithmic_bytes_per_step": nbytes}}


def run_spec_step_pooled(args, torch, gdn):
    """The speculative step over a fixed-state pool: verify reads each request's
    committed slot (capsule, no final state), replay writes the accepted prefix into
    its inactive slot in the same pool, and publication swaps the two slot arrays
    on the device. Same shapes as spec_verify_replay; the pool holds K disjoint
    slot sets (one committed/inactive pair of arrays each) rotated over steps so
    every step reads cold state."""
    from gdn_workloads import workload_inputs
    inp = workload_inputs("spec_verify_replay")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R, cap = len(inp["cu_seqlens"]) - 1, inp["capacity"]
    W = gdn.capsule_width(Hk, Hv, Dk, Dv)
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    acc_host = inp["accepted"]
    acc = _dev(acc_host, torch)
    state_bytes = R * Hv * Dv * Dk * 4
    sets = max(2, -(-(3 * BANK_TARGET_BYTES // 2) // (2 * state_bytes)))
    P = 2 * R * sets
    pool = torch.empty((P, Hv, Dv, Dk), dtype=torch.float32, device="cuda")
    init = _dev(inp["initial_state"], torch)
    pairs = []
    for j in range(sets):
        base = 2 * R * j
        committed = torch.arange(base, base + R, dtype=torch.int32, device="cuda")
        inactive = torch.arange(base + R, base + 2 * R, dtype=torch.int32, device="cuda")
        pool[base:base + R] = init
        pool[base + R:base + 2 * R] = init
        pairs.append((committed, inactive))
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    capsule = torch.empty((R, cap, W), dtype=torch.float32, device="cuda")
    host_cu = inp["cu_seqlens"]

    def step(i):
        committed, inactive = pairs[i % sets]
        gdn.gdn_forward_pooled(q, k, v, a, b, A_log, dt_bias, cu, out, num_slots=P, read_slots=committed,
                               write_slots=None, initial_state=pool, final_state=None,
                               state_update=capsule, state_update_capacity=cap, cu_seqlens_host=host_cu,
                               plan=gdn.PLAN_RECURRENT)
        gdn.gdn_replay_pooled(pool, capsule, acc, pool, num_k_heads=Hk, state_update_capacity=cap,
                              read_slots=committed, write_slots=inactive, accepted_host=acc_host)
        gdn.gdn_publish_slots(committed, inactive)

    _log(f"pooled verify+replay+publish: R={R} T=4 Hv={Hv} slots={P}")
    ms = _time_steps(torch, step, args.steps, args.warmup)
    per_call = _per_call(torch, step, 50, args.warmup + args.steps)
    io = 2
    verify_bytes = (state_bytes + R * cap * W * 4 + 2 * N * Hk * Dk * io + 2 * N * Hv * Dv * io
                    + 2 * N * Hv * 4 + 2 * Hv * 4 + (R + 1) * 4 + R * 4)
    replay_bytes = 2 * state_bytes + int(acc_host.sum()) * W * 4 + 3 * R * 4
    nbytes = verify_bytes + replay_bytes + 4 * R * 4
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "per_call": per_call,
            "config": {"requests": R, "draft_tokens": 4, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                       "capacity": cap, "accepted": acc_host.tolist(), "pool_slots": P},
            "roofline": {"bound": "hbm", "kernel": "gdn_capsule+gdn_replay+gdn_publish",
                         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("spec_step_pooled"),
                         "algorithmic_bytes_per_step": nbytes}}


def run_spec_step_pooled_fused(args, torch, gdn):
    """spec_step_pooled with the fused step: one gdn_replay_forward_pooled call (the
    previous step's accepted prefix replayed from each committed slot into its
    inactive slot, this step's verify from that state) and the publication, per
    step. Pool and slot sets as spec_step_pooled; two capsule buffers alternate."""
    from gdn_workloads import workload_inputs
    inp = workload_inputs("spec_verify_replay")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R, cap = len(inp["cu_seqlens"]) - 1, inp["capacity"]
    W = gdn.capsule_width(Hk, Hv, Dk, Dv)
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    acc_host = inp["accepted"]
    acc = _dev(acc_host, torch)
    state_bytes = R * Hv * Dv * Dk * 4
    sets = max(2, -(-(3 * BANK_TARGET_BYTES // 2) // (2 * state_bytes)))
    P = 2 * R * sets
    pool = torch.empty((P, Hv, Dv, Dk), dtype=torch.float32, device="cuda")
    init = _dev(inp["initial_state"], torch)
    pairs = []
    for j in range(sets):
        base = 2 * R * j
        committed = torch.arange(base, base + R, dtype=torch.int32, device="cuda")
        inactive = torch.arange(base + R, base + 2 * R, dtype=torch.int32, device="cuda")
        pool[base:base + R] = init
        pool[base + R:base + 2 * R] = init
        pairs.append((committed, inactive))
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    caps = [torch.empty((R, cap, W), dtype=torch.float32, device="cuda") for _ in range(2)]
    host_cu = inp["cu_seqlens"]
    # a real previous capsule for the first step
    gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=init, state_update=caps[1],
                    state_update_capacity=cap, cu_seqlens_host=host_cu, plan=gdn.PLAN_RECURRENT)

    def step(i):
        committed, inactive = pairs[i % sets]
        gdn.gdn_replay_forward_pooled(q, k, v, a, b, A_log, dt_bias, cu, out, num_slots=P, read_slots=committed,
                                      write_slots=inactive, initial_state=pool, replay_pool=pool,
                                      prev_state_update=caps[(i + 1) % 2], state_update=caps[i % 2],
                                      state_update_capacity=cap, accepted=acc, accepted_host=acc_host,
                                      cu_seqlens_host=host_cu, plan=gdn.PLAN_RECURRENT)
        gdn.gdn_publish_slots(committed, inactive)

    _log(f"pooled fused replay+verify+publish: R={R} T=4 Hv={Hv} slots={P}")
    ms = _time_steps(torch, step, args.steps, args.warmup)
    per_call = _per_call(torch, step, 50, args.warmup + args.steps)
    io = 2
    nbytes = (2 * state_bytes + int(acc_host.sum()) * W * 4 + R * cap * W * 4 + 2 * N * Hk * Dk * io
              + 2 * N * Hv * Dv * io + 2 * N * Hv * 4 + 2 * Hv * 4 + (R + 1) * 4 + R * 4 + 2 * R * 4
              + 4 * R * 4)
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "per_call": per_call,
            "config": {"requests": R, "draft_tokens": 4, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                       "capacity": cap, "accepted": acc_host.tolist(), "pool_slots": P},
            "roofline": {"bound": "hbm", "kernel": "gdn_replay_verify+gdn_publish",
                         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("spec_step_pooled_fused"),
                         "algorithmic_bytes_per_step": nbytes}}


def prefill_flops(lengths, Hk, Hv, D, chunk=64):
    """MFMA flops of the chunked prefill as the method computes it: per chunk of L
    tokens, Hk * 4 L^2 D (Q K^T and K K^T, once per key head) + Hv * (4 L^2 D +
    6 L D^2) per value head: U = T' (V - e^g rk X) and P U (two L x L x D
    products) and the three state contractions K S0^T, Q S0^T and U^T K (the
    reassociated WY form never forms W = T K). Triangular products count as full
    L x L; the fp32 triangular inverse (about 2 % more) is not counted."""
    total = 0
    for n in lengths:
        for c0 in range(0, int(n), chunk):
            L = min(chunk, int(n) - c0)
            total += Hk * 4 * L * L * D + Hv * (4 * L * L * D + 6 * L * D * D)
    return total


def prefill_flops_wy3(lengths, Hk, Hv, D, chunk=64):
    """The same count with all three L^2 D WY products per value head (W = T K
    formed explicitly), Hk 4 L^2 D + Hv (6 L^2 D + 6 L D^2) per chunk: reported
    beside the executed count for comparison with that convention."""
    total = 0
    for n in lengths:
        for c0 in range(0, int(n), chunk):
            L = min(chunk, int(n) - c0)
            total += Hk * 4 * L * L * D + Hv * (6 * L * L * D + 6 * L * D * D)
    return total


def run_prefill(args, torch, gdn, name):
    from gdn_workloads import workload_inputs
    inp = workload_inputs(name)
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R = len(inp["cu_seqlens"]) - 1
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    init = _dev(inp["initial_state"], torch)
    fin = torch.empty_like(init)
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    host_cu = inp["cu_seqlens"]
    nws = gdn.gdn_forward_workspace_bytes(N, R, Hk, Hv, Dk, Dv, gdn.GDN_F16, cu_seqlens_host=host_cu)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    plan = gdn.gdn_resolve_plan(N, R, Hk, Hv, Dk, Dv, gdn.GDN_F16, cu_seqlens_host=host_cu)

    def step(i):
        gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=init, final_state=fin,
                        cu_seqlens_host=host_cu, workspace=ws)

    # timed after at least 0.2 s of the same calls, over enough calls for 20 ms or more
    steps = max(20, args.steps // 5)
    warm = max(2, args.warmup // 10)
    _log(f"{name}: N={N} R={R} Hv={Hv} plan={'chunk' if plan == gdn.PLAN_CHUNK else 'recurrent'} steps={steps}")
    ms = _time_steps(torch, step, steps, warm, min_warm_s=0.2)
    per_call = _per_call(torch, step, 10, warm + steps)
    flops = prefill_flops(inp["lengths"], Hk, Hv, Dk)
    flops_wy3 = prefill_flops_wy3(inp["lengths"], Hk, Hv, Dk)
    io = 2
    nbytes = (2 * N * Hk * Dk * io + 2 * N * Hv * Dv * io + 2 * N * Hv * 4 + 2 * Hv * 4
              + (R + 1) * 4 + 2 * R * Hv * Dv * Dk * 4)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "per_call": per_call,
            "config": {"tokens": N, "requests": R, "lengths": [int(x) for x in inp["lengths"]],
                       "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv, "chunk": 64, "workspace_bytes": nws},
            "roofline": {"bound": "mfma", "kernel": "gdn_chunk_index+gdn_chunk_prep+gdn_chunk_scan",
                         "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": measured_traffic(name),
                         "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": nbytes,
                         "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "frac_three_wy_products": flops_wy3 / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}}


# ------------------------------------------------------- causal convolution
def conv_bytes(N, R, C, K, io, capture_rows=0) -> int:
    """Algorithmic HBM bytes of one convolution call: x read and output written
    once, the carried state read and the final state written once, the filter,
    bias and cu_seqlens read once, and the captured rows written."""
    return (2 * N * C * io + 2 * R * C * (K - 1) * 4 + C * K * 4 + C * 4 + (R + 1) * 4
            + capture_rows * C * 4)


def _time_graph(torch, step, steps, warmup, per_graph):
    """Average ms per step of `step(i)` when `per_graph` consecutive steps are
    replayed as one HIP graph (a call too short to time launch by launch)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(warmup):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            step(i)
    replays = max(1, -(-steps // per_graph))
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(replays):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / (replays * per_graph), replays * per_graph


def run_conv(args, torch, gdn, name):
    """The compact causal convolution upstream of the operator, C = 2 Hk Dk + Hv Dv
    = 8192 channels (Hk=16, Hv=32, D=128), K = 4, fp16 I/O, SiLU. conv_prefill: the
    ragged prefill lengths, final state to its own buffer; conv_decode: 64 requests x
    1 token, state updated in place over rotating banks, steps replayed as a HIP graph."""
    from gdn_workloads.conv import conv_channels, make_conv_inputs
    C, K = conv_channels(16, 32, 128, 128), 4
    if name == "conv_prefill":
        inp = make_conv_inputs(None, C, K, "f16", seed=3, num_drawn=8, max_drawn=4096)
    else:
        inp = make_conv_inputs([1] * 64, C, K, "f16", seed=1)
    N, R = inp["x"].shape[0], len(inp["lengths"])
    x, w, bias, cu = (_dev(inp[n], torch) for n in ("x", "weight", "bias", "cu_seqlens"))
    out = torch.empty_like(x)
    host_cu = inp["cu_seqlens"]
    state_bytes = R * C * (K - 1) * 4
    nbytes = conv_bytes(N, R, C, K, 2)
    if name == "conv_prefill":
        # x and the output are 251 MB each: with one copy, part of x is still in the
        # 256 MB Infinity Cache from the call before (76 against 92 us per call), so
        # the calls rotate over three copies of x, output and states
        banks = 3
        sets = [(x if j == 0 else x.clone(), out if j == 0 else torch.empty_like(x),
                 _dev(inp["initial_state"], torch), torch.empty_like(_dev(inp["initial_state"], torch)))
                for j in range(banks)]

        def step(i):
            xs, outs, init, fin = sets[i % banks]
            gdn.gdn_conv_forward(xs, w, bias, cu, outs, initial_state=init, final_state=fin,
                                 cu_seqlens_host=host_cu)

        _log(f"{name}: N={N} R={R} C={C} K={K}")
        ms = _time_steps(torch, step, max(20, args.steps // 5), max(5, args.warmup // 5), min_warm_s=0.2)
        timing = ("HIP events around consecutive calls, after at least 0.2 s of the same calls; "
                  "x, output and states rotate over three copies")
    else:
        banks = max(2, -(-BANK_TARGET_BYTES // state_bytes))
        states = [_dev(inp["initial_state"], torch) for _ in range(banks)]

        def step(i):
            s = states[i % banks]
            gdn.gdn_conv_forward(x, w, bias, cu, out, initial_state=s, final_state=s,
                                 cu_seqlens_host=host_cu)

        _log(f"{name}: R={R} C={C} K={K} banks={banks} (graph of {banks} steps)")
        ms, n = _time_graph(torch, step, args.steps, args.warmup, banks)
        timing = f"HIP events around graph replays, {n} steps"
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "config": {"tokens": N, "requests": R, "channels": C, "kernel_size": K,
                       "io_dtype": "f16", "activation": "silu", "state_banks": banks,
                       "timing": timing},
            "roofline": {"bound": "hbm", "kernel": "gdn_conv_forward", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(name), "algorithmic_bytes_per_step": nbytes}}


def run_conv_decode_fused(args, torch, gdn):
    """The batched decode step with its causal convolution fused in
    (gdn_conv_decode_forward): 64 requests x 1 token, Hk=16, Hv=32, D=128, fp16, the
    convolution over the 8192 concatenated q, k, v channels (K = 4, SiLU). The GDN
    state is updated in place over rotating banks; the convolution's carried inputs
    go from one bank to the next (they cannot be updated in place). Beside it, the
    same step as the two separate calls it replaces (gdn_conv_forward, then
    gdn_forward on contiguous q, k, v), timed the same way."""
    from gdn_workloads import workload_inputs
    from gdn_workloads.conv import conv_channels, make_conv_inputs
    inp = workload_inputs("batched_decode")
    N, Hk, Dk = inp["q"].shape
    Hv, Dv = inp["v"].shape[1:]
    R = len(inp["cu_seqlens"]) - 1
    C, K = conv_channels(Hk, Hv, Dk, Dv), 4
    cinp = make_conv_inputs([1] * R, C, K, "f16", seed=1)
    q, k, v, a, b = (_dev(inp[n], torch) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias, cu = _dev(inp["A_log"], torch), _dev(inp["dt_bias"], torch), _dev(inp["cu_seqlens"], torch)
    x, w, bias = (_dev(cinp[n], torch) for n in ("x", "weight", "bias"))
    state_bytes = R * Hv * Dv * Dk * 4
    n_banks = max(2, -(-BANK_TARGET_BYTES // state_bytes))
    banks = [_dev(inp["initial_state"], torch) for _ in range(n_banks)]
    cbanks = [_dev(cinp["initial_state"], torch) for _ in range(n_banks + 1)]
    out = torch.empty((N, Hv, Dv), dtype=q.dtype, device="cuda")
    y = torch.empty_like(x)
    host_cu = inp["cu_seqlens"]

    def fused(i):
        s = banks[i % n_banks]
        gdn.gdn_conv_decode_forward(x, w, bias, a, b, A_log, dt_bias, cu, out, num_k_heads=Hk, head_k_dim=Dk,
                                    conv_initial_state=cbanks[i % (n_banks + 1)],
                                    conv_final_state=cbanks[(i + 1) % (n_banks + 1)],
                                    initial_state=s, final_state=s, cu_seqlens_host=host_cu)

    def separate(i):
        s = banks[i % n_banks]
        cs = cbanks[i % (n_banks + 1)]
        gdn.gdn_conv_forward(x, w, bias, cu, y, initial_state=cs, final_state=cs, cu_seqlens_host=host_cu)
        gdn.gdn_forward(q, k, v, a, b, A_log, dt_bias, cu, out, initial_state=s, final_state=s,
                        cu_seqlens_host=host_cu, plan=gdn.PLAN_RECURRENT)

    _log(f"decode with the convolution fused: R={R} Hv={Hv} C={C} banks={n_banks}")
    ms = _time_steps(torch, fused, args.steps, args.warmup)
    ms_sep = _time_steps(torch, separate, args.steps, args.warmup)
    nbytes = (decode_bytes(inp) - 2 * N * Hk * Dk * 2 - N * Hv * Dv * 2      # q, k, v not read
              + N * C * 2 + 2 * R * C * (K - 1) * 4 + C * K * 4 + C * 4)     # x, carried inputs, filter
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"value": N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "config": {"tokens": N, "requests": R, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv, "io_dtype": "f16",
                       "channels": C, "kernel_size": K, "activation": "silu", "state_banks": n_banks,
                       "separate_calls_ms_per_step": ms_sep,
                       "separate_calls": "gdn_conv_forward (8192 channels, in place) + gdn_forward (decode)"},
            "roofline": {"bound": "hbm", "kernel": "gdn_conv_decode", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": measured_traffic("conv_decode_fused"),
                         "algorithmic_bytes_per_step": nbytes}}


def run_hbm_copy(args, torch):
    """Reference stream: device-to-device copies of 128 MiB fp32 buffers rotated over
    banks (read 128 MiB + write 128 MiB per step). Its known byte count calibrates
    the FETCH_SIZE / WRITE_SIZE counters, and its rate is the achievable HBM rate of
    a plain read+write stream."""
    n = 32 * 2 ** 20
    banks = max(2, -(-BANK_TARGET_BYTES // (n * 4)))
    src = [torch.randn(n, device="cuda") for _ in range(banks)]
    dst = [torch.empty_like(x) for x in src]
    ms = _time_steps(torch, lambda i: dst[i % banks].copy_(src[i % banks]), args.steps, args.warmup)
    nbytes = 2 * n * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"value": gbs, "unit": "GB/s", "ms_per_step": ms, "bytes_per_step": nbytes,
            "config": {"buffer_bytes": n * 4, "banks": banks},
            "roofline": {"bound": "hbm", "kernel": "copy", "achieved": gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="all",
                    choices=["all", "batched_decode", "spec_verify_replay", "ragged_prefill", "long_prefill",
                             "decode_effective_dense", "conv_prefill", "conv_decode",
                             "spec_step_pooled", "spec_step_fused", "spec_step_pooled_fused", "decode_kmajor",
                             "conv_decode_fused", "hbm_copy"],
                    help="all: the decode line plus the other workloads under 'workloads'")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="length of each oracle CPU-baseline sample (0 skips them)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator's sharding across GPUs is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gateddeltanet_recurrence_amd as gdn
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    gdn.lib()
    if args.workload not in ("all", "batched_decode"):
        fn = {"spec_verify_replay": lambda: run_verify_replay(args, torch, gdn),
              "ragged_prefill": lambda: run_prefill(args, torch, gdn, "ragged_prefill"),
              "long_prefill": lambda: run_prefill(args, torch, gdn, "long_prefill"),
              "decode_effective_dense": lambda: run_decode_effective_dense(args, torch, gdn),
              "conv_prefill": lambda: run_conv(args, torch, gdn, "conv_prefill"),
              "conv_decode": lambda: run_conv(args, torch, gdn, "conv_decode"),
              "spec_step_pooled": lambda: run_spec_step_pooled(args, torch, gdn),
              "spec_step_fused": lambda: run_spec_step_fused(args, torch, gdn),
              "spec_step_pooled_fused": lambda: run_spec_step_pooled_fused(args, torch, gdn),
              "decode_kmajor": lambda: run_decode_kmajor(args, torch, gdn),
              "conv_decode_fused": lambda: run_conv_decode_fused(args, torch, gdn),
              "hbm_copy": lambda: run_hbm_copy(args, torch)}[args.workload]
        res = fn()
        print(json.dumps({"metric": METRIC, "workload": args.workload, **res}), flush=True)
        return
    line, inp = run_decode(args, torch, gdn)
    if args.workload == "all":
        line["workloads"] = {
            "spec_verify_replay": run_verify_replay(args, torch, gdn),
            "ragged_prefill": run_prefill(args, torch, gdn, "ragged_prefill"),
            "long_prefill": run_prefill(args, torch, gdn, "long_prefill"),
            "decode_effective_dense": run_decode_effective_dense(args, torch, gdn),
            "conv_prefill": run_conv(args, torch, gdn, "conv_prefill"),
            "conv_decode": run_conv(args, torch, gdn, "conv_decode"),
            "spec_step_pooled": run_spec_step_pooled(args, torch, gdn),
            "spec_step_fused": run_spec_step_fused(args, torch, gdn),
            "spec_step_pooled_fused": run_spec_step_pooled_fused(args, torch, gdn),
            "decode_kmajor": run_decode_kmajor(args, torch, gdn),
            "conv_decode_fused": run_conv_decode_fused(args, torch, gdn),
        }
    if args.cpu_seconds > 0:
        from gdn_workloads import workload_inputs
        _log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s per workload")
        from oracle.cpu_baseline import cpu_baseline
        line["cpu_baseline"] = cpu_baseline(inp, "decode", args.cpu_seconds)
        if args.workload == "all":
            wl = line["workloads"]
            wl["spec_verify_replay"]["cpu_baseline"] = cpu_baseline(
                workload_inputs("spec_verify_replay"), "verify_replay", args.cpu_seconds)
            for name in ("ragged_prefill", "long_prefill"):
                wl[name]["cpu_baseline"] = cpu_baseline(workload_inputs(name), "prefill", args.cpu_seconds,
                                                        max_tokens=8192)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
