"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop counts the
roofline fractions are computed from, the hash check that keeps a counted
traffic figure only while its kernel sources are unchanged, and the refusal of
more than one GPU.

Expected values are written out from the definitions: the decode moves the FP32
state once each way plus q, k, v, output, gates and cu_seqlens; the prefill
counts, per chunk of L tokens, Hk 4 L^2 D for Q K^T and K K^T per key head and
Hv (4 L^2 D + 6 L D^2) per value head (two L x L products and three state
contractions), and beside it the count with a third L x L product.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_bytes_of_the_batched_decode(bench):
    from gdn_workloads import workload_inputs
    inp = workload_inputs("batched_decode")
    state = 2 * 64 * 32 * 128 * 128 * 4                   # read and written once
    io = 2 * 64 * 16 * 128 * 2 + 2 * 64 * 32 * 128 * 2    # q, k; v, output (fp16)
    gates = 2 * 64 * 32 * 4 + 2 * 32 * 4 + 65 * 4         # a, b; A_log, dt_bias; cu_seqlens
    assert bench.decode_bytes(inp) == state + io + gates == 270_025_220


def test_prefill_flops_per_chunk(bench):
    Hk, Hv, D = 16, 48, 128

    def chunk(L):        # executed: Q K^T, K K^T per key head; T'Z, PU and 3 state products per value head
        return Hk * 4 * L * L * D + Hv * (4 * L * L * D + 6 * L * D * D)

    def chunk_wy3(L):    # with W = T K formed as well
        return Hk * 4 * L * L * D + Hv * (6 * L * L * D + 6 * L * D * D)

    assert bench.prefill_flops([64], Hk, Hv, D) == chunk(64)
    # a request of 65 tokens is a full chunk and a chunk of one; chunks never span requests
    assert bench.prefill_flops([65, 1], Hk, Hv, D) == chunk(64) + 2 * chunk(1)
    assert bench.prefill_flops([0], Hk, Hv, D) == 0
    # the long prefill: 512 chunks of 64
    assert bench.prefill_flops([32768], Hk, Hv, D) == 512 * chunk(64) == 223_338_299_392
    assert bench.prefill_flops_wy3([32768], Hk, Hv, D) == 512 * chunk_wy3(64) == 249_108_103_168


def test_conv_bytes(bench):
    N, R, C, K, io = 10, 2, 8, 4, 2
    x_out = 2 * N * C * io
    state = 2 * R * C * (K - 1) * 4
    params = C * K * 4 + C * 4 + (R + 1) * 4
    assert bench.conv_bytes(N, R, C, K, io) == x_out + state + params
    assert bench.conv_bytes(N, R, C, K, io, capture_rows=3) == x_out + state + params + 3 * C * 4


def test_traffic_figure_kept_only_for_unchanged_sources(bench, monkeypatch):
    # every timed workload carries a counter figure, valid while its kernels' sources are
    for wl in ("batched_decode", "decode_effective_dense", "decode_kmajor", "spec_verify_replay",
               "spec_step_fused", "spec_step_pooled", "ragged_prefill", "long_prefill", "conv_prefill",
               "conv_decode"):
        rec = bench.MEASURED_TRAFFIC[wl]
        assert bench.measured_traffic(wl) in (rec["bytes"], None), wl
    rec = dict(bench.MEASURED_TRAFFIC["batched_decode"])
    stale = dict(rec, sha256_16="0" * 16)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, "batched_decode", stale)
    assert bench.measured_traffic("batched_decode") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")   # no JSON line


def test_cpu_baseline_times_the_oracle_on_every_head():
    # a tiny workload, two worker processes: the slowest head group sets the rate
    from gdn_workloads import make_inputs
    from oracle.cpu_baseline import cpu_baseline
    inp = make_inputs([3, 5], 1, 4, 8, 8, "f32", seed=3)
    res = cpu_baseline(inp, "prefill", 0.05)
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s" and res["value"] > 0
    assert 1 <= res["cores"] <= 4 and "4 value heads" in res["sample"]
