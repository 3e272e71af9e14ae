"""GPU checks of gdn_replay_forward, the speculative step in one pass over the
committed state: replay of the previous step's accepted capsule prefix into the
inactive bank, then the verify of this step's drafts from that state.

The fused call must write the same bytes as gdn_replay followed by gdn_forward
from the replayed bank (bit for bit: both run the same arithmetic in the same
order), leave the committed bank untouched, and match the float64 oracle
(gdn_replay, then gdn_forward) within the usual tolerances: FP32 I/O rel-max
1e-4; FP16 I/O output max-abs 2e-2 and state relative L2 1e-3; capsule alpha
and k^ 1e-5, u 1e-3 (FP16) against the largest entry.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs, workload_inputs
from gpu_helpers import assert_parity, dev, device_inputs, rel_max, rel_l2

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


def _step_inputs(lengths, Hk, Hv, Dk, Dv, io, cap, seed):
    """This step's drafts, a previous capsule (a real one: the verify of earlier
    drafts from the committed bank, on the GPU) and accepted counts."""
    inp = make_inputs(lengths, Hk, Hv, Dk, Dv, io, seed=seed, capacity=cap)
    prev_inp = make_inputs([cap] * len(lengths), Hk, Hv, Dk, Dv, io, seed=seed + 1, capacity=cap)
    prev_inp["initial_state"] = inp["initial_state"]
    d = device_inputs(prev_inp, torch)
    W = gdn.capsule_width(Hk, Hv, Dk, Dv)
    R = len(lengths)
    prev = torch.full((R, cap, W), -7.0, dtype=torch.float32, device="cuda")
    out = torch.empty((sum(len_ for len_ in [cap] * R), Hv, Dv), dtype=d["v"].dtype, device="cuda")
    gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                    initial_state=d["initial_state"], state_update=prev, state_update_capacity=cap,
                    cu_seqlens_host=prev_inp["cu_seqlens"])
    rng = np.random.default_rng(seed + 2)
    accepted = rng.integers(0, cap + 1, R).astype(np.int32)
    return inp, prev, accepted


def _separate(d, inp, prev, acc, cap, fin):
    R, Hv, Dv, Dk = inp["initial_state"].shape
    dst = torch.full_like(d["initial_state"], float("nan"))
    gdn.gdn_replay(d["initial_state"], prev, acc, dst, num_k_heads=inp["Hk"], state_update_capacity=cap)
    W = gdn.capsule_width(inp["Hk"], Hv, Dk, Dv)
    capsule = torch.full((R, cap, W), -7.0, dtype=torch.float32, device="cuda")
    out = torch.full((inp["v"].shape[0], Hv, Dv), float("nan"), dtype=d["v"].dtype, device="cuda")
    gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                    initial_state=dst, final_state=fin, state_update=capsule, state_update_capacity=cap,
                    cu_seqlens_host=inp["cu_seqlens"])
    return dst, out, capsule


def _fused(d, inp, prev, acc, acc_host, cap, fin):
    R, Hv, Dv, Dk = inp["initial_state"].shape
    dst = torch.full_like(d["initial_state"], float("nan"))
    W = gdn.capsule_width(inp["Hk"], Hv, Dk, Dv)
    capsule = torch.full((R, cap, W), -7.0, dtype=torch.float32, device="cuda")
    out = torch.full((inp["v"].shape[0], Hv, Dv), float("nan"), dtype=d["v"].dtype, device="cuda")
    gdn.gdn_replay_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"],
                           out, initial_state=d["initial_state"], final_state=fin, state_update=capsule,
                           state_update_capacity=cap, cu_seqlens_host=inp["cu_seqlens"],
                           prev_state_update=prev, accepted=acc, replay_state=dst, accepted_host=acc_host)
    return dst, out, capsule


@pytest.mark.parametrize("io,Dk,Dv,lengths,final", [
    ("f16", 128, 128, [4] * 16, False),            # the speculative verify shape (Hv = 48 below)
    ("f16", 128, 128, [4, 0, 3, 1, 4], True),
    ("f32", 64, 32, [2, 4, 0, 3], True),
    ("f32", 16, 16, [1, 4, 4], False),
    ("f16", 128, 16, [4, 2, 0, 3], True),          # rows past Dv in the one wave of a head
])
def test_fused_step_equals_separate_calls(io, Dk, Dv, lengths, final):
    cap = 4
    Hk, Hv = (16, 48) if len(lengths) == 16 else (2, 4)
    inp, prev, accepted = _step_inputs(lengths, Hk, Hv, Dk, Dv, io, cap, seed=950 + Dk + len(lengths))
    _case(f"fused step {io} Dk={Dk} Dv={Dv} lengths={lengths} accepted={accepted.tolist()} final={final}")
    d = device_inputs(inp, torch)
    acc = dev(accepted, torch)
    committed = d["initial_state"].clone()
    fin_a = torch.full_like(committed, float("nan")) if final else None
    fin_b = torch.full_like(committed, float("nan")) if final else None
    dst_a, out_a, cap_a = _separate(d, inp, prev, acc, cap, fin_a)
    dst_b, out_b, cap_b = _fused(d, inp, prev, acc, accepted, cap, fin_b)
    torch.cuda.synchronize()
    assert torch.equal(d["initial_state"], committed)                 # committed bank untouched
    assert torch.equal(dst_a, dst_b)
    assert torch.equal(out_a, out_b)
    assert torch.equal(cap_a, cap_b)
    if final:
        assert torch.equal(fin_a, fin_b)

    # against the oracle: the replayed bank, then the verify from it
    ref_dst = O.gdn_replay(inp["initial_state"], prev.cpu().numpy(), accepted, Hk, Hv, Dk, Dv)
    got_dst = dst_b.cpu().numpy()
    if io == "f32":
        assert rel_max(got_dst, ref_dst) <= 1e-5
    else:
        assert rel_l2(got_dst, ref_dst) <= 1e-5
    W = O.capsule_width(Hk, Hv, Dk, Dv)
    ref_o, ref_s, ref_cap = O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                                          inp["dt_bias"], inp["cu_seqlens"], got_dst,
                                          state_update_capacity=cap,
                                          state_update_init=np.full((len(lengths), cap, W), -7.0))
    assert_parity(io, out_b.cpu().numpy(), ref_o, fin_b.cpu().numpy() if final else None,
                  ref_s if final else None, "fused step")
    got = cap_b.cpu().numpy()
    sa, sk, sd = O.capsule_sections(Hk, Hv, Dk, Dv)
    tol_u = 1e-4 if io == "f32" else 1e-3
    for r, L in enumerate(lengths):
        assert np.all(got[r, L:] == -7.0)
        if L:
            assert rel_max(got[r, :L, sa], ref_cap[r, :L, sa]) <= 1e-5
            assert rel_max(got[r, :L, sk], ref_cap[r, :L, sk]) <= 1e-5
            assert rel_max(got[r, :L, sd], ref_cap[r, :L, sd]) <= tol_u


def test_fused_step_device_counts_beyond_capacity():
    # accepted read on the device only (no mirror), values past either end of
    # [0, capacity]: clamped as gdn_replay does
    cap = 4
    lengths = [3, 4, 2, 4]
    inp, prev, _ = _step_inputs(lengths, 2, 4, 128, 128, "f16", cap, seed=990)
    accepted = np.array([9, -3, 4, 0], np.int32)
    _case(f"fused step device counts {accepted.tolist()}")
    d = device_inputs(inp, torch)
    acc = dev(accepted, torch)
    dst_a, out_a, cap_a = _separate(d, inp, prev, acc, cap, None)
    dst_b, out_b, cap_b = _fused(d, inp, prev, acc, None, cap, None)
    torch.cuda.synchronize()
    assert torch.equal(dst_a, dst_b) and torch.equal(out_a, out_b) and torch.equal(cap_a, cap_b)
    ref_dst = O.gdn_replay(inp["initial_state"], prev.cpu().numpy(), accepted, 2, 4, 128, 128)
    assert rel_l2(dst_b.cpu().numpy(), ref_dst) <= 1e-5
    # accepted 0 copies the committed rows exactly
    assert torch.equal(dst_b[3], d["initial_state"][3]) and torch.equal(dst_b[1], d["initial_state"][1])


def test_fused_step_spec_workload_chain():
    # three steps of the speculative workload, each replaying the previous
    # step's capsule: fused and separate chains stay bit-identical
    inp = workload_inputs("spec_verify_replay")
    cap = inp["capacity"]
    Hk, Hv, Dk, Dv = inp["Hk"], inp["Hv"], inp["Dk"], inp["Dv"]
    d = device_inputs(inp, torch)
    R = len(inp["cu_seqlens"]) - 1
    W = gdn.capsule_width(Hk, Hv, Dk, Dv)
    rng = np.random.default_rng(996)
    bank_a, bank_b = d["initial_state"].clone(), d["initial_state"].clone()
    prev_a = torch.zeros((R, cap, W), dtype=torch.float32, device="cuda")
    prev_b = prev_a.clone()
    for step in range(3):
        accepted = rng.integers(0, cap + 1, R).astype(np.int32)
        acc = dev(accepted, torch)
        if step == 0:
            accepted[:] = 0
            acc.zero_()
        _case(f"spec chain step {step} accepted={accepted.tolist()}")
        d_a = dict(d, initial_state=bank_a)
        dst_a, _, cap_a = _separate(d_a, inp, prev_a, acc, cap, None)
        d_b = dict(d, initial_state=bank_b)
        dst_b, _, cap_b = _fused(d_b, inp, prev_b, acc, accepted, cap, None)
        torch.cuda.synchronize()
        assert torch.equal(dst_a, dst_b) and torch.equal(cap_a, cap_b), step
        bank_a, bank_b, prev_a, prev_b = dst_a, dst_b, cap_a, cap_b


def _i32(x):
    return torch.tensor(np.asarray(x, np.int32), device="cuda")


@pytest.mark.parametrize("one_pool", [True, False])
def test_fused_step_pooled_equals_separate_calls(one_pool):
    # committed and inactive slots of one pool (or two pools); request 5's write
    # slot is -1: its replayed state is not written, its verify still runs
    R, cap, Hk, Hv, D = 6, 4, 2, 4, 128
    lengths = [4, 4, 3, 4, 0, 2]
    inp, prev, accepted = _step_inputs(lengths, Hk, Hv, D, D, "f16", cap, seed=1010)
    P = 2 * R
    rng = np.random.default_rng(1011)
    committed_np = rng.permutation(P)[:R].astype(np.int32)
    inactive_np = np.array([s for s in range(P) if s not in set(committed_np.tolist())], np.int32)
    rng.shuffle(inactive_np)
    inactive_np[5] = -1
    pool_np = rng.standard_normal((P, Hv, D, D)).astype(np.float32) * np.float32(0.05)
    pool_np[committed_np] = inp["initial_state"]
    d = device_inputs(inp, torch)
    W = gdn.capsule_width(Hk, Hv, D, D)
    acc = dev(accepted, torch)
    _case(f"fused pooled step one_pool={one_pool} accepted={accepted.tolist()}")

    def run(fused):
        pool = dev(pool_np, torch)
        dst_pool = pool if one_pool else dev(pool_np, torch)
        capsule = torch.full((R, cap, W), -7.0, dtype=torch.float32, device="cuda")
        out = torch.full((inp["v"].shape[0], Hv, D), float("nan"), dtype=torch.float16, device="cuda")
        common = dict(state_update=capsule, state_update_capacity=cap, cu_seqlens_host=inp["cu_seqlens"])
        if fused:
            gdn.gdn_replay_forward_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                          d["cu_seqlens"], out, num_slots=P, read_slots=_i32(committed_np),
                                          write_slots=_i32(inactive_np), read_slots_host=committed_np,
                                          write_slots_host=inactive_np, initial_state=pool,
                                          prev_state_update=prev, accepted=acc, accepted_host=accepted,
                                          replay_pool=dst_pool, **common)
        else:
            gdn.gdn_replay_pooled(pool, prev, acc, dst_pool, num_k_heads=Hk, state_update_capacity=cap,
                                  read_slots=_i32(committed_np), write_slots=_i32(inactive_np),
                                  read_slots_host=committed_np, write_slots_host=inactive_np,
                                  accepted_host=accepted)
            # the verify of request 5 (no written slot) reads the replay the fused call
            # keeps in registers: give the separate call that state through a scratch pool
            scratch = torch.zeros((R, Hv, D, D), dtype=torch.float32, device="cuda")
            gdn.gdn_replay(d["initial_state"], prev, acc, scratch, num_k_heads=Hk, state_update_capacity=cap)
            gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"],
                            out, initial_state=scratch, **common)
        torch.cuda.synchronize()
        return pool, dst_pool, out, capsule

    pa, da, oa, ca = run(False)
    pb, db, ob, cb = run(True)
    assert torch.equal(oa, ob) and torch.equal(ca, cb)
    assert torch.equal(da, db)
    got = db.cpu().numpy()
    # committed slots untouched; the slot of the request without a write slot too
    assert np.array_equal(pb.cpu().numpy()[committed_np], inp["initial_state"])
    untouched = [s for s in range(P) if s not in set(inactive_np.tolist())]
    assert np.array_equal(got[untouched], pool_np[untouched])
    ref = O.gdn_replay(inp["initial_state"], prev.cpu().numpy(), accepted, Hk, Hv, D, D)
    for r in range(R):
        if inactive_np[r] >= 0:
            assert rel_l2(got[inactive_np[r]], ref[r]) <= 1e-5, r
