"""GPU parity of the recurrent kernels (gdn_decode, gdn_capsule) and gdn_replay
against the float64 oracle, called through the C ABI.

Tolerances (written here, applied by gpu_helpers.assert_parity):
  FP32 I/O  max|x-y| / max|y| <= 1e-4 for output and final state
  FP16 I/O  output max-abs <= 2e-2, final-state relative L2 <= 1e-3
  replay vs the GPU's own recurrence on the same prefix: rel-max <= 1e-5
  capsule / accepted-prefix indexing: bit-exact (untouched rows keep their poison)
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from gdn_workloads import cu_from_lengths, make_inputs, workload_inputs
from gpu_helpers import (TOL_F32_REL, TOL_REPLAY_REL, assert_parity, dev, effective_gate_inputs,
                         oracle_forward,
                         rel_max, run_forward)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import gdn_oracle as O                   # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()                                         # fails loudly if libgdn.so is missing


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def test_tiny_recurrent_fp32():
    inp = workload_inputs("tiny_recurrent")
    _case("tiny_recurrent fp32 T=16 Hk=Hv=2 D=16")
    res = run_forward(inp, torch, gdn)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f32", res["output"], ref_o, res["final_state"], ref_s, "tiny")


def test_batched_decode_in_place_fp16():
    inp = workload_inputs("batched_decode")
    _case("batched_decode fp16 R=64 Hv=32 D=128 in place")
    res = run_forward(inp, torch, gdn, in_place=True)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "decode")


@pytest.mark.parametrize("io", ["f32", "f16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
def test_ragged_recurrent_shapes(io, Dk, Dv):
    lengths = [1, 7, 0, 33, 5, 64, 2]
    inp = make_inputs(lengths, 2, 6, Dk, Dv, io, seed=100 + Dk + Dv)
    _case(f"ragged recurrent io={io} Dk={Dk} Dv={Dv} lengths={lengths}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_RECURRENT)
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity(io, res["output"], ref_o, res["final_state"], ref_s, f"{io} {Dk}x{Dv}")


def test_explicit_scale_and_zero_initial_state():
    inp = make_inputs([9, 4], 1, 2, 32, 32, "f32", seed=7, initial="zero")
    _case("explicit scale 0.3, zero initial state")
    res = run_forward(inp, torch, gdn, scale=0.3)
    ref_o, ref_s, _ = oracle_forward(inp, O, scale=0.3)
    assert rel_max(res["output"], ref_o) <= TOL_F32_REL
    assert rel_max(res["final_state"], ref_s) <= TOL_F32_REL


def test_in_place_matches_out_of_place_bitwise():
    inp = make_inputs([3, 1, 6], 2, 4, 128, 128, "f16", seed=8)
    _case("in place vs out of place")
    a = run_forward(inp, torch, gdn)
    b = run_forward(inp, torch, gdn, in_place=True)
    assert np.array_equal(a["output"], b["output"])
    assert np.array_equal(a["final_state"], b["final_state"])


def test_packing_invariance_bitwise():
    lengths = [17, 5, 40]                              # a small ragged mix
    inp = make_inputs(lengths, 2, 4, 64, 64, "f16", seed=9)
    _case(f"packing invariance lengths={lengths}")
    packed = run_forward(inp, torch, gdn, plan=gdn.PLAN_RECURRENT)
    cu = inp["cu_seqlens"]
    for r, L in enumerate(lengths):
        sub = dict(inp)
        for n in ("q", "k", "v", "a", "b"):
            sub[n] = inp[n][cu[r]:cu[r + 1]]
        sub["cu_seqlens"] = cu_from_lengths([L])
        sub["initial_state"] = inp["initial_state"][r:r + 1]
        alone = run_forward(sub, torch, gdn, plan=gdn.PLAN_RECURRENT)
        assert np.array_equal(alone["output"], packed["output"][cu[r]:cu[r + 1]])
        assert np.array_equal(alone["final_state"][0], packed["final_state"][r])


def test_no_final_state_leaves_initial_untouched():
    inp = make_inputs([4, 4], 1, 2, 128, 128, "f16", seed=10)
    _case("final_state NULL")
    res = run_forward(inp, torch, gdn, write_final=False)
    assert np.array_equal(res["initial_after"], inp["initial_state"])
    ref_o, _, _ = oracle_forward(inp, O)
    assert_parity("f16", res["output"], ref_o, what="no-final")


def test_empty_segments_copy_state():
    inp = make_inputs([0, 3, 0, 0], 1, 1, 32, 16, "f32", seed=11)
    _case("empty segments")
    res = run_forward(inp, torch, gdn)
    for r in (0, 2, 3):
        assert np.array_equal(res["final_state"][r], inp["initial_state"][r])


@pytest.mark.parametrize("io,capacity", [("f32", 0), ("f16", 4)])
def test_no_tokens_at_all(io, capacity):
    # N = 0 with requests: every segment is empty, so the final state is the
    # initial one (bit for bit) and, with a capsule, no capsule row is written
    inp = make_inputs([0, 0, 0], 2, 4, 128, 64, io, seed=12, capacity=capacity)
    _case(f"no tokens {io} capacity={capacity}")
    res = run_forward(inp, torch, gdn, capacity=capacity, poison=-7.0)
    assert res["output"].shape[0] == 0
    assert np.array_equal(res["final_state"], inp["initial_state"])
    if capacity:
        assert np.all(res["state_update"] == -7.0)


def test_bf16_rejected_without_writes():
    inp = make_inputs([2], 1, 1, 16, 16, "f32", seed=12)
    _case("bf16 rejected")
    d = {n: dev(inp[n], torch) for n in ("a", "b", "A_log", "dt_bias", "cu_seqlens")}
    q = dev(inp["q"], torch, torch.bfloat16)
    k = dev(inp["k"], torch, torch.bfloat16)
    v = dev(inp["v"], torch, torch.bfloat16)
    out = torch.full(v.shape, 3.0, dtype=torch.bfloat16, device="cuda")
    st = gdn.gdn_forward(q, k, v, d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                         check=False)
    torch.cuda.synchronize()
    assert st == gdn.GDN_ERR_DTYPE
    assert bool(torch.all(out == 3.0))


# ---------------------------------------------------------------- capsule
def _capsule_sections(Hk, Hv, Dk, Dv):
    return O.capsule_sections(Hk, Hv, Dk, Dv)


def test_spec_verify_capsule():
    inp = workload_inputs("spec_verify_replay")
    cap = inp["capacity"]
    _case("spec_verify capsule R=16 T=4 Hv=48 cap=4")
    res = run_forward(inp, torch, gdn, capacity=cap, write_final=False, poison=-7.0)
    ref_o, _, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0)
    assert_parity("f16", res["output"], ref_o, what="verify")
    assert np.array_equal(res["initial_after"], inp["initial_state"])   # committed bank untouched
    got = res["state_update"]
    sa, sk, sd = _capsule_sections(inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"])
    assert rel_max(got[..., sa], ref_cap[..., sa]) <= 1e-5
    assert rel_max(got[..., sk], ref_cap[..., sk]) <= 1e-5
    # deltas depend on the state the way outputs do: FP16-input tolerance on their scale
    assert rel_max(got[..., sd], ref_cap[..., sd]) <= 1e-3


def test_capture_count_and_untouched_rows():
    lengths = [4, 2, 5, 0, 3]
    cap = 4
    inp = make_inputs(lengths, 2, 4, 64, 32, "f32", seed=13, capacity=cap)
    cc = np.array([4, 4, 2, 3, 0], np.int32)
    _case(f"capture_count {cc.tolist()} lengths={lengths}")
    res = run_forward(inp, torch, gdn, capacity=cap, capture_count=cc, poison=-7.0)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, capacity=cap, capture_count=cc, poison=-7.0)
    assert_parity("f32", res["output"], ref_o, res["final_state"], ref_s, "capture")
    got = res["state_update"]
    for r, L in enumerate(lengths):
        n = min(L, cc[r], cap)
        assert np.all(got[r, n:] == -7.0), r                    # bit-exact: untouched
        assert np.all(got[r, :n] != -7.0), r
        if n:
            assert rel_max(got[r, :n], ref_cap[r, :n]) <= TOL_F32_REL


@pytest.mark.parametrize("Dk,Dv,lengths", [(16, 16, [16]), (16, 16, [21, 6]), (32, 16, [40])])
def test_capsule_small_heads_vs_oracle(Dk, Dv, lengths):
    # one-wave workgroups (small Dv) stage a group of up to 16 tokens in several
    # passes; every captured value and every output is checked, not just coverage
    cap = max(lengths)
    inp = make_inputs(lengths, 2, 2, Dk, Dv, "f32", seed=16, capacity=cap)
    _case(f"capsule Dk={Dk} Dv={Dv} lengths={lengths}")
    res = run_forward(inp, torch, gdn, capacity=cap, poison=-7.0)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0)
    assert_parity("f32", res["output"], ref_o, res["final_state"], ref_s, "capsule small heads")
    got = res["state_update"]
    for r, L in enumerate(lengths):
        assert np.all(got[r, L:] == -7.0)
        assert rel_max(got[r, :L], ref_cap[r, :L]) <= TOL_F32_REL


# ------------------------------------------------ gate and layout variants
@pytest.mark.parametrize("io", ["f32", "f16"])
def test_effective_gates_vs_oracle(io):
    inp = effective_gate_inputs(make_inputs([9, 1, 0, 17], 2, 4, 64, 32, io, seed=17), seed=18)
    _case(f"effective gates {io}")
    res = run_forward(inp, torch, gdn, gate="none", plan=gdn.PLAN_RECURRENT)
    ref_o, ref_s, _ = oracle_forward(inp, O, gate="none")
    assert_parity(io, res["output"], ref_o, res["final_state"], ref_s, f"effective gates {io}")


def test_effective_gates_capsule():
    cap = 4
    inp = effective_gate_inputs(make_inputs([4, 3, 6], 2, 4, 128, 128, "f16", seed=19, capacity=cap),
                                seed=20)
    _case("effective gates capsule")
    res = run_forward(inp, torch, gdn, gate="none", capacity=cap, poison=-7.0)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, gate="none", capacity=cap, poison=-7.0)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, "effective gates capsule")
    sa, sk, sd = O.capsule_sections(inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"])
    got = res["state_update"]
    assert np.array_equal(got[..., sa], ref_cap[..., sa].astype(np.float32))   # clamped alpha, exact
    assert rel_max(got[..., sd], ref_cap[..., sd]) <= 1e-3


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (32, 64)])
def test_capsule_deep_decay_vs_oracle(Dk, Dv):
    # decays spread over twelve decades (and exact 0s and 1s) drive the running
    # product of a segment's decays far below any fixed floor within a few
    # tokens, so the staged recurrence both keeps it factored out of the state
    # and folds it back in, many times per segment
    lengths = [40, 23, 1, 0]
    cap = max(lengths)
    inp = make_inputs(lengths, 2, 4, Dk, Dv, "f32", seed=22, capacity=cap)
    inp = effective_gate_inputs(inp, seed=23)
    rng = np.random.default_rng(24)
    alpha = 10.0 ** rng.uniform(-12.0, 0.0, inp["a"].shape)
    alpha.flat[::7] = 1.0
    alpha.flat[3::11] = 0.0
    inp["a"] = alpha.astype(np.float32)
    _case(f"capsule deep decay Dk={Dk} Dv={Dv} lengths={lengths}")
    res = run_forward(inp, torch, gdn, gate="none", capacity=cap, poison=-7.0)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, gate="none", capacity=cap, poison=-7.0)
    assert_parity("f32", res["output"], ref_o, res["final_state"], ref_s, "capsule deep decay")
    got = res["state_update"]
    for r, L in enumerate(lengths):
        assert np.all(got[r, L:] == -7.0)
        if L:
            assert rel_max(got[r, :L], ref_cap[r, :L]) <= TOL_F32_REL


@pytest.mark.parametrize("io,capacity", [("f32", 0), ("f16", 0), ("f16", 4)])
def test_dense_layout_equals_packed_bitwise(io, capacity):
    inp = make_inputs([5, 5, 5], 2, 4, 128, 64, io, seed=21, capacity=capacity)
    _case(f"dense layout {io} capacity={capacity}")
    packed = run_forward(inp, torch, gdn, capacity=capacity, poison=-7.0)
    dense = run_forward(inp, torch, gdn, capacity=capacity, poison=-7.0, dense=True)
    for key in ("output", "final_state") + (("state_update",) if capacity else ()):
        assert np.array_equal(dense[key], packed[key]), key


def test_dense_rank4_tensors_through_the_binding():
    # [R, S, H, D] tensors straight into the binding (no cu_seqlens)
    R, S, Hk, Hv, D = 3, 6, 2, 4, 32
    inp = make_inputs([S] * R, Hk, Hv, D, D, "f32", seed=22)
    _case("dense rank-4 binding")
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
    q4, k4 = d["q"].reshape(R, S, Hk, D), d["k"].reshape(R, S, Hk, D)
    v4 = d["v"].reshape(R, S, Hv, D)
    out4 = torch.empty_like(v4)
    fin = torch.empty((R, Hv, D, D), dtype=torch.float32, device="cuda")
    init = dev(inp["initial_state"], torch)
    gdn.gdn_forward(q4, k4, v4, d["a"].reshape(R, S, Hv), d["b"].reshape(R, S, Hv), d["A_log"],
                    d["dt_bias"], None, out4, initial_state=init, final_state=fin)
    torch.cuda.synchronize()
    ref_o, ref_s, _ = oracle_forward(inp, O)
    assert_parity("f32", out4.reshape(R * S, Hv, D).cpu().numpy(), ref_o, fin.cpu().numpy(), ref_s,
                  "dense rank-4")


def test_capture_count_clamped_to_capacity():
    # counts beyond capacity capture capacity rows, negative counts none; the
    # values are the oracle's, which clamps the same way (a pinned reading)
    inp = make_inputs([6, 6, 2], 1, 2, 16, 16, "f32", seed=14, capacity=3)
    cc = np.array([99, -5, 99], np.int32)
    _case("capture_count clamped [99, -5, 99] at capacity 3")
    res = run_forward(inp, torch, gdn, capacity=3, capture_count=cc, poison=-7.0)
    ref_o, ref_s, ref_cap = oracle_forward(inp, O, capacity=3, capture_count=cc, poison=-7.0)
    assert_parity("f32", res["output"], ref_o, res["final_state"], ref_s, "clamped capture")
    got = res["state_update"]
    for r, n in enumerate([3, 0, 2]):
        assert np.all(got[r, n:] == -7.0), r                    # bit-exact: untouched
        assert np.all(ref_cap[r, n:] == -7.0), r
        if n:
            assert rel_max(got[r, :n], ref_cap[r, :n]) <= TOL_F32_REL


# ----------------------------------------------------------------- replay
def _replay(src, capsule, accepted, Hk, cap, accepted_host=True):
    s = torch.from_numpy(np.ascontiguousarray(src)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(capsule)).cuda()
    a = torch.from_numpy(np.ascontiguousarray(accepted)).cuda()
    dst = torch.full_like(s, float("nan"))
    gdn.gdn_replay(s, c, a, dst, num_k_heads=Hk, state_update_capacity=cap,
                   accepted_host=accepted if accepted_host else None)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


def test_replay_matches_own_recurrence_and_oracle():
    inp = workload_inputs("spec_verify_replay")
    cap, Hk, Hv, Dk, Dv = inp["capacity"], inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"]
    acc = inp["accepted"]
    _case(f"replay accepted={acc.tolist()}")
    verify = run_forward(inp, torch, gdn, capacity=cap, write_final=False)
    dst = _replay(inp["initial_state"], verify["state_update"], acc, Hk, cap)
    # the GPU's own sequential state after the accepted prefix of every request
    cu = inp["cu_seqlens"]
    sub = dict(inp)
    idx = np.concatenate([np.arange(cu[r], cu[r] + acc[r]) for r in range(len(acc))]).astype(int)
    for n in ("q", "k", "v", "a", "b"):
        sub[n] = inp[n][idx]
    sub["cu_seqlens"] = cu_from_lengths(acc)
    own = run_forward(sub, torch, gdn, plan=gdn.PLAN_RECURRENT)
    assert rel_max(dst, own["final_state"]) <= TOL_REPLAY_REL
    # and the float64 oracle replay of the GPU capsule
    ref = O.gdn_replay(inp["initial_state"], verify["state_update"], acc, Hk, Hv, Dk, Dv)
    assert rel_max(dst, ref) <= TOL_REPLAY_REL
    for r in np.nonzero(acc == 0)[0]:
        assert np.array_equal(dst[r], inp["initial_state"][r])      # m = 0 copies exactly


@pytest.mark.parametrize("m", [0, 1, 2, 3, 4])
def test_replay_every_prefix_length(m):
    lengths = [4, 4, 4]
    inp = make_inputs(lengths, 2, 4, 128, 64, "f16", seed=15, capacity=4)
    _case(f"replay prefix m={m}")
    verify = run_forward(inp, torch, gdn, capacity=4, write_final=False)
    acc = np.full(3, m, np.int32)
    dst = _replay(inp["initial_state"], verify["state_update"], acc, 2, 4, accepted_host=False)
    ref = O.gdn_replay(inp["initial_state"], verify["state_update"], acc, 2, 4, 128, 64)
    assert rel_max(dst, ref) <= TOL_REPLAY_REL
    if m == 0:
        assert np.array_equal(dst, inp["initial_state"])


def test_replay_clamps_device_accepted_without_mirror():
    # no host mirror: the kernel clamps accepted to [0, capacity] itself (a bounds
    # check in the kernel; -3 replays nothing, cap + 5 replays the capacity rows)
    cap, Hk, Hv, Dk, Dv = 4, 2, 4, 128, 64
    inp = make_inputs([4, 4, 4], Hk, Hv, Dk, Dv, "f16", seed=17, capacity=cap)
    _case("replay device accepted [-3, 9, 2], no host mirror")
    verify = run_forward(inp, torch, gdn, capacity=cap, write_final=False)
    acc = np.array([-3, cap + 5, 2], np.int32)
    dst = _replay(inp["initial_state"], verify["state_update"], acc, Hk, cap, accepted_host=False)
    ref = O.gdn_replay(inp["initial_state"], verify["state_update"], acc, Hk, Hv, Dk, Dv)
    assert rel_max(dst, ref) <= TOL_REPLAY_REL
    assert np.array_equal(dst[0], inp["initial_state"][0])           # clamped to 0: a copy
    # the capacity rows replayed equal the GPU's own recurrence over those tokens
    own = run_forward(inp, torch, gdn, plan=gdn.PLAN_RECURRENT)
    assert rel_max(dst[1], own["final_state"][1]) <= TOL_REPLAY_REL


def test_replay_rejects_accepted_beyond_capacity():
    src = np.zeros((2, 2, 16, 16), np.float32)
    capsule = np.zeros((2, 4, gdn.capsule_width(1, 2, 16, 16)), np.float32)
    s = torch.from_numpy(src).cuda()
    c = torch.from_numpy(capsule).cuda()
    a = torch.tensor([1, 5], dtype=torch.int32, device="cuda")
    dst = torch.full_like(s, 9.0)
    st = gdn.gdn_replay(s, c, a, dst, num_k_heads=1, state_update_capacity=4,
                        accepted_host=[1, 5], check=False)
    torch.cuda.synchronize()
    assert st == gdn.GDN_ERR_CAPACITY and bool(torch.all(dst == 9.0))
