"""GPU parity of the verify kernel (gdn_capsule: capsule capture, fp16 I/O,
Dk = Dv = 128, V-major) against the float64 oracle, called through the C ABI,
on what the speculative verify workload does not reach: segments longer than
one staged group of tokens, final states (in place too; an empty request's
comes back bit for bit), no initial state with
every update rule, capture counts past either end of [0, capacity], state rows
over a wide range of magnitudes, and heads with fewer value rows (Dv = 16, 32)
than one wave holds.

Tolerances (as for every fp16 path): output max-abs <= 2e-2, final state
relative L2 <= 1e-3; capsule alpha and k^ rel-max <= 1e-5, u <= 1e-3; untouched
capsule rows bit-exact. The row-scale case sets v = 0, so every delta is the
state's own product and is compared per row at 1e-4 of that row's largest.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs
from gpu_helpers import assert_parity, oracle_forward, rel_max, run_forward

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import gdn_oracle as O                   # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def _check_capsule(got, ref, inp, n_per_request):
    sa, sk, sd = O.capsule_sections(inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"])
    for r, n in enumerate(n_per_request):
        assert np.all(got[r, n:] == -7.0), r                     # untouched rows keep the poison
        if n:
            assert rel_max(got[r, :n, sa], ref[r, :n, sa]) <= 1e-5, r
            assert rel_max(got[r, :n, sk], ref[r, :n, sk]) <= 1e-5, r
            assert rel_max(got[r, :n, sd], ref[r, :n, sd]) <= 1e-3, r


@pytest.mark.parametrize("in_place", [False, True])
def test_verify_several_passes_with_final_state(in_place):
    lengths = [20, 9, 8, 1, 0, 16, 17]
    cap = 20
    inp = make_inputs(lengths, 2, 4, 128, 128, "f16", seed=900, capacity=cap)
    _case(f"verify passes lengths={lengths} in_place={in_place}")
    res = run_forward(inp, torch, gdn, capacity=cap, in_place=in_place, poison=-7.0,
                      plan=gdn.PLAN_RECURRENT)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "verify passes")
    _check_capsule(res["state_update"], ref_cap, inp, lengths)
    for r, L in enumerate(lengths):
        # no tokens: every row of the initial state comes back bit for bit (the rows
        # a wave's second pass holds are loaded on this path only)
        if L == 0:
            assert np.array_equal(res["final_state"][r], np.asarray(inp["initial_state"])[r]), r


def test_verify_zero_initial_state_and_rules():
    lengths = [11, 3, 5]
    cap = 8
    for rule in ("gated_delta", "delta", "gated", "linear"):
        inp = make_inputs(lengths, 2, 6, 128, 128, "f16", seed=901, initial="zero", capacity=cap)
        _case(f"verify zero state rule={rule}")
        res = run_forward(inp, torch, gdn, capacity=cap, poison=-7.0, rule=rule, plan=gdn.PLAN_RECURRENT)
        ref_o, ref_s, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0, rule=rule)
        assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, f"verify zero state {rule}")
        _check_capsule(res["state_update"], ref_cap, inp, [min(L, cap) for L in lengths])


def test_verify_capture_counts_clamped():
    lengths = [12, 5, 9, 8, 3]
    cap = 8
    cc = np.array([99, -5, 3, 8, 0], np.int32)
    inp = make_inputs(lengths, 2, 4, 128, 128, "f16", seed=902, capacity=cap)
    _case(f"verify capture_count {cc.tolist()}")
    res = run_forward(inp, torch, gdn, capacity=cap, capture_count=cc, write_final=False, poison=-7.0)
    ref_o, _, ref_cap = oracle_forward(inp, O, capacity=cap, capture_count=cc, poison=-7.0)
    assert_parity("f16", res["output"], ref_o, what="verify capture counts")
    n = [min(L, max(int(c), 0), cap) for L, c in zip(lengths, cc)]
    _check_capsule(res["state_update"], ref_cap, inp, n)


def test_verify_state_rows_over_wide_range():
    # rows of the initial state scaled by 2^e, e from -70 to +12; v = 0 makes
    # each delta the state's own product, so a lost digit shows per row
    lengths = [6, 4]
    cap = 6
    inp = make_inputs(lengths, 2, 4, 128, 128, "f16", seed=903, capacity=cap)
    rng = np.random.default_rng(904)
    e = rng.integers(-70, 13, size=inp["initial_state"].shape[:3])
    inp["initial_state"] = (inp["initial_state"] * np.exp2(e)[..., None]).astype(np.float32)
    inp["v"] = np.zeros_like(inp["v"])
    _case("verify wide row range")
    res = run_forward(inp, torch, gdn, capacity=cap, write_final=False, poison=-7.0)
    _, _, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0)
    sa, sk, sd = O.capsule_sections(inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"])
    got = res["state_update"]
    Hv, Dv = inp["Hv"], inp["Dv"]
    for r, L in enumerate(lengths):
        d_got = got[r, :L, sd].reshape(L, Hv, Dv)
        d_ref = ref_cap[r, :L, sd].reshape(L, Hv, Dv)
        assert np.all(np.isfinite(d_got))
        # per (head, row): error against that row's largest delta over the tokens
        scale = np.abs(d_ref).max(axis=0)
        err = np.abs(d_got - d_ref).max(axis=0)
        nz = scale > 0
        assert np.all(err[nz] <= 1e-4 * scale[nz]), float((err[nz] / scale[nz]).max())
        assert rel_max(got[r, :L, sa], ref_cap[r, :L, sa]) <= 1e-5


@pytest.mark.parametrize("io", ["f16", "f32"])
@pytest.mark.parametrize("Dv", [16, 32])
def test_verify_rows_past_dv(io, Dv):
    # Dk = 128 with Dv below one wave's 32 state rows: the lanes whose rows lie
    # past Dv must write neither output nor delta (their range-checked stores are
    # dropped); the rows that exist match the oracle
    lengths = [4, 3, 0, 4, 1]
    cap = 4
    inp = make_inputs(lengths, 2, 4, 128, Dv, io, seed=910 + Dv, capacity=cap)
    _case(f"verify rows past Dv io={io} Dk=128 Dv={Dv} lengths={lengths}")
    res = run_forward(inp, torch, gdn, capacity=cap, poison=-7.0, plan=gdn.PLAN_RECURRENT)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0)
    assert_parity(io, res["output"], ref_o, res["final_state"], ref_s, f"verify Dv={Dv}")
    _check_capsule(res["state_update"], ref_cap, inp, lengths)
