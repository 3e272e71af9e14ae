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
host's cores on a bounded sample of the same workload.
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
METRIC = "GDN tokens/s + achieved HBM GB/s (decode/replay), MFMA % (prefill)"
BANK_TARGET_BYTES = 512 * 2 ** 20

# HBM traffic of the dominant kernel, from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# runs of this workload (KiB per dispatch, scaled by the copy-kernel calibration).
# None until measured for the current kernel.
MEASURED_TRAFFIC = {}


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
    traffic = MEASURED_TRAFFIC.get("gdn_decode")
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
                     "avg_kernel_us": ms_step * 1e3},
    }
    return line, inp


def cpu_baseline_decode(inp, seconds):
    """The float64 oracle as it stands, on this host: consecutive decode steps of
    the same workload, each starting from the previous step's final state."""
    from threadpoolctl import threadpool_limits
    from oracle import gdn_oracle as O
    state = inp["initial_state"].astype(np.float64)
    n_steps = 0
    N = inp["q"].shape[0]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            _, state, _ = O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                                        inp["dt_bias"], inp["cu_seqlens"], state)
            n_steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": n_steps * N / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_steps} consecutive decode steps of the batched_decode workload "
                      f"({N} tokens each) in {el:.1f} s, numpy float64, 1 thread; host has "
                      f"{os.cpu_count()} logical CPUs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="batched_decode", choices=["batched_decode"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="length of the oracle CPU-baseline sample (0 skips it)")
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
    line, inp = run_decode(args, torch, gdn)
    if args.cpu_seconds > 0:
        _log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline_decode(inp, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
