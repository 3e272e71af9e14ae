"""GPU parity of the chunked prefill (gdn_chunk_index / _prep / _scan) against
the float64 oracle, called through the C ABI with the CHUNK plan.

Tolerances (FP16 I/O): output max-abs <= 2e-2, final-state relative L2 <= 1e-3.
Packing, host-mirror and in-place invariances are bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import cu_from_lengths, make_inputs, workload_inputs
from gpu_helpers import (assert_parity, effective_gate_inputs, max_abs, oracle_forward,
                         oracle_forward_all_heads, rel_l2, run_forward, sample_heads_inputs)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import gdn_oracle as O                   # noqa: E402

RAGGED = [1, 63, 64, 65, 130, 0, 200, 7]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.mark.parametrize("Hk,Hv", [(2, 4), (1, 3), (2, 2), (1, 6)])
def test_chunk_ragged_vs_oracle(Hk, Hv):
    inp = make_inputs(RAGGED, Hk, Hv, 128, 128, "f16", seed=40 + Hv)
    _case(f"chunk ragged Hk={Hk} Hv={Hv} lengths={RAGGED}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, f"chunk G={Hv // Hk}")


@pytest.mark.parametrize("host_cu", [True, False])
def test_chunk_no_tokens_at_all(host_cu):
    # N = 0 with requests, forced CHUNK: no chunk to prepare, every scan workgroup
    # walks zero chunks and writes back the initial state (bit for bit); without a
    # host mirror the workspace is sized by the bound, not by the (zero) count
    inp = make_inputs([0, 0, 0], 2, 4, 128, 128, "f16", seed=52)
    _case(f"chunk no tokens host_cu={host_cu}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK, host_cu=host_cu)
    assert res["output"].shape[0] == 0
    assert np.array_equal(res["final_state"], inp["initial_state"])


def test_chunk_matches_forced_recurrent():
    inp = make_inputs([300, 64, 129], 2, 4, 128, 128, "f16", seed=41)
    _case("chunk vs recurrent")
    ch = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    rc = run_forward(inp, torch, gdn, plan=gdn.PLAN_RECURRENT)
    assert max_abs(ch["output"], rc["output"]) <= 2e-2
    assert rel_l2(ch["final_state"], rc["final_state"]) <= 1e-3


def test_chunk_zero_initial_state_and_no_final():
    inp = make_inputs([70, 5], 1, 2, 128, 128, "f16", seed=42, initial="zero")
    _case("chunk zero initial state")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "chunk zero-init")
    inp2 = make_inputs([70, 5], 1, 2, 128, 128, "f16", seed=42)
    res2 = run_forward(inp2, torch, gdn, plan=gdn.PLAN_CHUNK, write_final=False)
    assert np.array_equal(res2["initial_after"], inp2["initial_state"])


def test_chunk_packing_invariance_bitwise():
    lengths = [100, 17, 64]
    inp = make_inputs(lengths, 2, 4, 128, 128, "f16", seed=43)
    _case(f"chunk packing invariance {lengths}")
    packed = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    cu = inp["cu_seqlens"]
    for r, L in enumerate(lengths):
        sub = dict(inp)
        for n in ("q", "k", "v", "a", "b"):
            sub[n] = inp[n][cu[r]:cu[r + 1]]
        sub["cu_seqlens"] = cu_from_lengths([L])
        sub["initial_state"] = inp["initial_state"][r:r + 1]
        alone = run_forward(sub, torch, gdn, plan=gdn.PLAN_CHUNK)
        assert np.array_equal(alone["output"], packed["output"][cu[r]:cu[r + 1]])
        assert np.array_equal(alone["final_state"][0], packed["final_state"][r])


# 16 key heads x group 2: 4 or more requests give enough workgroups for the
# 64-row scan tiles
WIDE = dict(Hk=16, Hv=32)


def test_chunk_wide_tiles_vs_oracle():
    inp = make_inputs(RAGGED, WIDE["Hk"], WIDE["Hv"], 128, 128, "f16", seed=46)
    _case(f"chunk 64-row tiles Hk={WIDE['Hk']} Hv={WIDE['Hv']} lengths={RAGGED}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "chunk 64-row tiles")


def test_chunk_wide_tiles_few_requests_vs_oracle():
    lengths = [200, 1, 64, 97]                      # 4 x 16 x 2 heads x 2 tiles = 256 workgroups
    inp = make_inputs(lengths, WIDE["Hk"], WIDE["Hv"], 128, 128, "f16", seed=48)
    _case(f"chunk 64-row tiles Hk={WIDE['Hk']} Hv={WIDE['Hv']} lengths={lengths}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "chunk 64-row tiles, 4 requests")


@pytest.mark.parametrize("lengths", [[130, 64, 1, 200, 65, 9, 128, 70], [300, 2, 129, 64]])
def test_chunk_tile_width_invariance_bitwise(lengths):
    # with 16 key heads x group 2 the batch runs the 64-row scan tiles, a request
    # alone the 32-row ones; each 16-row block of the state goes through the same
    # arithmetic in both
    inp = make_inputs(lengths, WIDE["Hk"], WIDE["Hv"], 128, 128, "f16", seed=47)
    _case(f"chunk tile width invariance {lengths}")
    packed = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    cu = inp["cu_seqlens"]
    for r in sorted({0, len(lengths) // 2, len(lengths) - 1}):
        sub = dict(inp)
        for n in ("q", "k", "v", "a", "b"):
            sub[n] = inp[n][cu[r]:cu[r + 1]]
        sub["cu_seqlens"] = cu_from_lengths([lengths[r]])
        sub["initial_state"] = inp["initial_state"][r:r + 1]
        alone = run_forward(sub, torch, gdn, plan=gdn.PLAN_CHUNK)
        assert np.array_equal(alone["output"], packed["output"][cu[r]:cu[r + 1]])
        assert np.array_equal(alone["final_state"][0], packed["final_state"][r])


def test_chunk_effective_gates_vs_oracle():
    # effective gates with exact state resets (alpha = 0) inside chunks, and
    # values past [0, 1] that both sides clamp
    inp = effective_gate_inputs(make_inputs(RAGGED, 2, 4, 128, 128, "f16", seed=49), seed=50)
    _case(f"chunk effective gates lengths={RAGGED}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK, gate="none")
    ref_o, ref_s, _ = oracle_forward(inp, O, gate="none")
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "chunk effective gates")


def test_chunk_dense_layout_equals_packed_bitwise():
    inp = make_inputs([130, 130, 130], 2, 4, 128, 128, "f16", seed=51)
    _case("chunk dense layout")
    packed = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    dense = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK, dense=True)
    assert np.array_equal(dense["output"], packed["output"])
    assert np.array_equal(dense["final_state"], packed["final_state"])


def test_chunk_without_host_mirror_is_identical():
    inp = make_inputs([90, 1, 0, 40], 1, 2, 128, 128, "f16", seed=44)
    _case("chunk host mirror vs none")
    a = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    b = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK, host_cu=False)
    assert np.array_equal(a["output"], b["output"])
    assert np.array_equal(a["final_state"], b["final_state"])


def test_chunk_in_place_bitwise():
    inp = make_inputs([77, 3], 1, 2, 128, 128, "f16", seed=45)
    _case("chunk in place")
    a = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    b = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK, in_place=True)
    assert np.array_equal(a["output"], b["output"])
    assert np.array_equal(a["final_state"], b["final_state"])


def test_chunk_strong_decay_stays_finite():
    inp = make_inputs([200], 1, 2, 128, 128, "f16", seed=46)
    inp["A_log"] = np.log(np.full(2, 16.0, np.float32))
    inp["a"] = inp["a"] + np.float32(4.0)
    _case("chunk strong decay")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert np.all(np.isfinite(res["output"])) and np.all(np.isfinite(res["final_state"]))
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "strong decay")


def test_chunk_plan_refused_for_fp32_io():
    inp = make_inputs([80], 1, 1, 128, 128, "f32", seed=47)
    with pytest.raises(gdn.GDNError) as ei:
        run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK)
    assert ei.value.status == gdn.GDN_ERR_PLAN
    # AUTO falls back to the recurrent kernels for fp32 I/O
    assert gdn.gdn_resolve_plan(80, 1, 1, 1, 128, 128, gdn.GDN_F32) == gdn.PLAN_RECURRENT


@pytest.mark.parametrize("name", ["ragged_prefill", "long_prefill"])
def test_full_size_prefill_vs_oracle(name):
    """Full-size workload on the GPU (every head, the AUTO plan and launch shape the
    bench times), checked against the float64 recurrence on every value head over
    every token (head groups in parallel CPU worker processes)."""
    inp = workload_inputs(name)
    Hv = inp["Hv"]
    _case(f"{name} full size N={inp['q'].shape[0]} Hv={Hv}, oracle on all heads")
    assert gdn.gdn_resolve_plan(inp["q"].shape[0], len(inp["lengths"]), inp["Hk"], Hv, 128, 128,
                                cu_seqlens_host=inp["cu_seqlens"]) == gdn.PLAN_CHUNK
    res = run_forward(inp, torch, gdn)
    ref_o, ref_s = oracle_forward_all_heads(inp)
    for h in range(Hv):
        assert_parity("f16", res["output"][:, h], ref_o[:, h], res["final_state"][:, h], ref_s[:, h],
                      f"{name} head {h}")
