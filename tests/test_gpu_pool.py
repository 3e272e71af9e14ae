"""GPU parity of the pooled fixed-state entry points (gdn_forward_pooled,
gdn_replay_pooled, gdn_conv_forward_pooled, gdn_conv_replay_pooled,
gdn_publish_slots) against the float64 pooled oracle, called through the C ABI.

Tolerances: as for the request-indexed calls (FP32 I/O 1e-4 relative; FP16 I/O
output max-abs 2e-2, state rel-L2 1e-3; replay vs the GPU's own recurrence 1e-5
relative; convolution states bit-exact). Slot handling is exact: every slot a
call does not write keeps its bytes, and publication swaps the slot arrays.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs
from gdn_workloads.conv import make_conv_inputs
from gpu_helpers import TOL_REPLAY_REL, assert_parity, dev, rel_max

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import conv_oracle as CO                 # noqa: E402
from oracle import pool_oracle as PO                 # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def _i32(x):
    return torch.tensor(np.asarray(x, np.int32), dtype=torch.int32, device="cuda")


def _fwd_args(inp):
    return [inp[n] for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")]


def _gpu_forward_pooled(inp, pool_np, rd, wr, *, P, host_slots=True, same_pool=True, plan=None,
                        capacity=0, out_pool_np=None):
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    N, Hv, Dv = inp["v"].shape
    R = len(inp["cu_seqlens"]) - 1
    Hk, Dk = inp["Hk"], inp["Dk"]
    pool = dev(pool_np.astype(np.float32), torch)
    out_pool = pool if same_pool else dev(out_pool_np.astype(np.float32), torch)
    out = torch.full((N, Hv, Dv), float("nan"), dtype=d["v"].dtype, device="cuda")
    su = None
    if capacity:
        su = torch.zeros((R, capacity, gdn.capsule_width(Hk, Hv, Dk, Dv)), device="cuda")
    io = gdn.GDN_F16 if inp["io_dtype"] == "f16" else gdn.GDN_F32
    plan = gdn.PLAN_AUTO if plan is None else plan
    nws = gdn.gdn_forward_workspace_bytes(N, R, Hk, Hv, Dk, Dv, io, capacity=capacity, plan=plan,
                                          cu_seqlens_host=inp["cu_seqlens"])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    gdn.gdn_forward_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"],
                           out, num_slots=P, read_slots=None if rd is None else _i32(rd),
                           write_slots=None if wr is None else _i32(wr),
                           read_slots_host=rd if host_slots and rd is not None else None,
                           write_slots_host=wr if host_slots and wr is not None else None,
                           initial_state=pool, final_state=out_pool, state_update=su,
                           state_update_capacity=capacity, cu_seqlens_host=inp["cu_seqlens"], plan=plan,
                           workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), out_pool.cpu().numpy(), su


def _check_pool(io, got_pool, ref_pool, written, what):
    untouched = [s for s in range(ref_pool.shape[0]) if s not in set(written)]
    assert np.array_equal(got_pool[untouched], ref_pool[untouched].astype(np.float32)), f"{what}: untouched slots"
    w = sorted(set(written))
    if w:
        assert_parity(io, np.zeros(1), np.zeros(1), got_pool[w], ref_pool[w], what)


@pytest.mark.parametrize("io", ["f32", "f16"])
def test_decode_pooled_double_buffer(io):
    R, P = 12, 30
    inp = make_inputs([1] * R, 2, 4, 64, 64, io, seed=400)
    rng = np.random.default_rng(1)
    pool = rng.standard_normal((P, 4, 64, 64)) * 0.05
    slots = rng.permutation(P)
    rd = slots[:R].copy()
    rd[3] = -1                                        # a new request: zero state
    wr = slots[R:2 * R].copy()
    wr[5] = -1                                        # verify-like: no write for this one
    _case(f"decode pooled {io} R={R} P={P}")
    o, got, _ = _gpu_forward_pooled(inp, pool, rd, wr, P=P, plan=gdn.PLAN_RECURRENT)
    o_ref, ref, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool.astype(np.float32), rd, wr)
    assert_parity(io, o, o_ref, what="pooled decode output")
    _check_pool(io, got, ref, [s for s in wr if s >= 0], "pooled decode")


def test_decode_pooled_in_place_and_identity():
    R = 8
    inp = make_inputs([2] * R, 2, 4, 32, 32, "f32", seed=401)
    rng = np.random.default_rng(2)
    pool = rng.standard_normal((R + 3, 4, 32, 32)) * 0.05
    rd = wr = rng.permutation(R + 3)[:R]               # every request updates its own slot
    _case("decode pooled in place")
    o, got, _ = _gpu_forward_pooled(inp, pool, rd, wr, P=R + 3, plan=gdn.PLAN_RECURRENT)
    o_ref, ref, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool.astype(np.float32), rd, wr)
    assert_parity("f32", o, o_ref, what="in place output")
    _check_pool("f32", got, ref, list(wr), "in place")
    _case("decode pooled identity slots (NULL arrays)")
    o, got, _ = _gpu_forward_pooled(inp, pool, None, None, P=R + 3, plan=gdn.PLAN_RECURRENT)
    o_ref, ref, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool.astype(np.float32), None, None)
    assert_parity("f32", o, o_ref, what="identity output")
    _check_pool("f32", got, ref, list(range(R)), "identity")


def test_chunk_pooled_separate_pools():
    lengths = [130, 64, 1, 200]
    R, P = len(lengths), 9
    inp = make_inputs(lengths, 1, 3, 128, 128, "f16", seed=402)
    rng = np.random.default_rng(3)
    pool_in = rng.standard_normal((P, 3, 128, 128)) * 0.05
    pool_out = rng.standard_normal((P, 3, 128, 128))
    rd = np.array([7, -1, 2, 2])                        # two requests may read one slot
    wr = np.array([0, 2, 8, 7])                         # disjoint pools: any distinct slots
    _case("chunk pooled fp16, separate read and write pools")
    o, got, _ = _gpu_forward_pooled(inp, pool_in, rd, wr, P=P, same_pool=False, plan=gdn.PLAN_CHUNK,
                                    out_pool_np=pool_out)
    o_ref, ref, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool_in.astype(np.float32), rd, wr,
                                          out_pool=pool_out.astype(np.float32))
    assert_parity("f16", o, o_ref, what="chunk pooled output")
    _check_pool("f16", got, ref, list(wr), "chunk pooled")


def test_device_slots_out_of_range_without_mirrors():
    R, P = 6, 8
    inp = make_inputs([1] * R, 1, 2, 16, 16, "f32", seed=403)
    pool = np.random.default_rng(4).standard_normal((P, 2, 16, 16)) * 0.05
    rd = np.array([0, 99, -5, 3, -1, 1])                # out of range: zero state
    wr = np.array([4, 5, 1000, 6, -7, 7])               # out of range: not written
    _case("pooled decode, device slots out of range, no mirrors")
    o, got, _ = _gpu_forward_pooled(inp, pool, rd, wr, P=P, host_slots=False, plan=gdn.PLAN_RECURRENT)
    o_ref, ref, _ = PO.gdn_forward_pooled(*_fwd_args(inp), pool.astype(np.float32), rd, wr)
    assert_parity("f32", o, o_ref, what="out-of-range slots")
    _check_pool("f32", got, ref, [4, 5, 6, 7], "out-of-range slots")


def test_speculative_step_verify_replay_publish():
    # committed slots -> verify (capsule, no final) -> replay the accepted prefix
    # into the inactive slots -> publish; the committed state is then the state
    # after exactly the accepted tokens
    T, R, cap = 4, 6, 4
    inp = make_inputs([T] * R, 2, 4, 64, 64, "f16", seed=404, capacity=cap)
    Hk, Hv, D = 2, 4, 64
    P = 2 * R
    rng = np.random.default_rng(5)
    committed_np = rng.permutation(P)[:R]
    inactive_np = np.array([s for s in range(P) if s not in set(committed_np)])
    rng.shuffle(inactive_np)
    pool_np = np.zeros((P, Hv, D, D), np.float32)
    pool_np[committed_np] = inp["initial_state"]
    accepted_np = np.array([0, 1, 2, 3, 4, 2], np.int32)
    committed, inactive = _i32(committed_np), _i32(inactive_np)
    pool = dev(pool_np, torch)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    out = torch.empty((T * R, Hv, D), dtype=torch.float16, device="cuda")
    su = torch.zeros((R, cap, gdn.capsule_width(Hk, Hv, D, D)), device="cuda")
    _case("pooled verify + replay + publish")
    gdn.gdn_forward_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"],
                           out, num_slots=P, read_slots=committed, write_slots=None,
                           initial_state=pool, final_state=None, state_update=su,
                           state_update_capacity=cap, cu_seqlens_host=inp["cu_seqlens"],
                           plan=gdn.PLAN_RECURRENT)
    gdn.gdn_replay_pooled(pool, su, _i32(accepted_np), pool, num_k_heads=Hk, state_update_capacity=cap,
                          read_slots=committed, write_slots=inactive, read_slots_host=committed_np,
                          write_slots_host=inactive_np, accepted_host=accepted_np)
    gdn.gdn_publish_slots(committed, inactive)
    torch.cuda.synchronize()
    new_committed = committed.cpu().numpy()
    assert np.array_equal(new_committed, inactive_np) and np.array_equal(inactive.cpu().numpy(), committed_np)
    got = pool.cpu().numpy()
    # the old committed slots are untouched
    assert np.array_equal(got[committed_np], inp["initial_state"])
    # against the GPU's own recurrence over the accepted prefix (request-indexed call)
    for r in range(R):
        m, t0 = int(accepted_np[r]), int(inp["cu_seqlens"][r])
        if m == 0:
            assert np.array_equal(got[new_committed[r]], inp["initial_state"][r])
            continue
        sl = slice(t0, t0 + m)
        s0 = dev(inp["initial_state"][r:r + 1], torch)
        fin = torch.empty_like(s0)
        o1 = torch.empty((m, Hv, D), dtype=torch.float16, device="cuda")
        gdn.gdn_forward(d["q"][sl], d["k"][sl], d["v"][sl], d["a"][sl], d["b"][sl], d["A_log"], d["dt_bias"],
                        _i32([0, m]), o1, initial_state=s0, final_state=fin, cu_seqlens_host=[0, m],
                        plan=gdn.PLAN_RECURRENT)
        torch.cuda.synchronize()
        err = rel_max(got[new_committed[r]], fin.cpu().numpy()[0])
        assert err <= TOL_REPLAY_REL, f"request {r}: replay vs recurrence {err:.3e}"


def test_conv_pooled_step():
    T, R, cap, C, K = 4, 5, 4, 1100, 4
    inp = make_conv_inputs([T] * R, C, K, "f16", seed=405, capacity=cap)
    P = 2 * R + 1
    rng = np.random.default_rng(6)
    perm = rng.permutation(P)
    committed_np, inactive_np = perm[:R], perm[R:2 * R]
    pool_np = rng.standard_normal((P, C, K - 1)).astype(np.float32)
    pool_np[committed_np] = inp["initial_state"]
    accepted_np = np.array([0, 4, 1, 3, 2], np.int32)
    pool = dev(pool_np, torch)
    committed, inactive = _i32(committed_np), _i32(inactive_np)
    x = dev(inp["x"], torch)
    out = torch.empty_like(x)
    su = torch.zeros((R, cap, C), device="cuda")
    _case("conv pooled verify + replay + publish")
    gdn.gdn_conv_forward_pooled(x, dev(inp["weight"], torch), dev(inp["bias"], torch),
                                dev(inp["cu_seqlens"], torch), out, num_slots=P, read_slots=committed,
                                write_slots=None, initial_state=pool, final_state=None, state_update=su,
                                state_update_capacity=cap, cu_seqlens_host=inp["cu_seqlens"])
    gdn.gdn_conv_replay_pooled(pool, su, _i32(accepted_np), pool, state_update_capacity=cap,
                               read_slots=committed, write_slots=inactive, read_slots_host=committed_np,
                               write_slots_host=inactive_np, accepted_host=accepted_np)
    gdn.gdn_publish_slots(committed, inactive)
    torch.cuda.synchronize()
    o_ref, _, cap_ref = PO.conv_forward_pooled(inp["x"], inp["weight"], inp["bias"], inp["cu_seqlens"],
                                               pool_np, committed_np, [-1] * R, state_update_capacity=cap)
    assert np.max(np.abs(out.float().cpu().numpy() - o_ref)) <= 2e-2
    assert np.array_equal(su.cpu().numpy(), cap_ref.astype(np.float32))
    ref_pool = PO.conv_replay_pooled(pool_np, cap_ref, accepted_np, committed_np, inactive_np)
    assert np.array_equal(pool.cpu().numpy(), ref_pool.astype(np.float32))
    assert np.array_equal(committed.cpu().numpy(), inactive_np)
    # the published state equals a forward over the accepted prefix
    got = pool.cpu().numpy()
    for r in range(R):
        m, t0 = int(accepted_np[r]), int(inp["cu_seqlens"][r])
        _, fin, _ = CO.conv_forward(inp["x"][t0:t0 + m], inp["weight"], inp["bias"], [0, m],
                                    inp["initial_state"][r:r + 1])
        assert np.array_equal(got[inactive_np[r]], fin[0].astype(np.float32)), r


def test_conv_pooled_forward_in_place_spanning():
    # long requests spanning workgroups, each updating its own slot in one pool
    lengths = [700, 3, 0, 1500]
    R, P, C, K = 4, 7, 1028, 4
    inp = make_conv_inputs(lengths, C, K, "f32", seed=406)
    rng = np.random.default_rng(7)
    pool_np = rng.standard_normal((P, C, K - 1)).astype(np.float32)
    rd = wr = np.array([5, 0, 3, 6])
    pool = dev(pool_np, torch)
    x = dev(inp["x"], torch)
    out = torch.empty_like(x)
    _case("conv pooled in place, spanning requests")
    gdn.gdn_conv_forward_pooled(x, dev(inp["weight"], torch), dev(inp["bias"], torch),
                                dev(inp["cu_seqlens"], torch), out, num_slots=P, read_slots=_i32(rd),
                                write_slots=_i32(wr), read_slots_host=rd, write_slots_host=wr,
                                initial_state=pool, final_state=pool, cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, ref_pool, _ = PO.conv_forward_pooled(inp["x"], inp["weight"], inp["bias"], inp["cu_seqlens"],
                                                pool_np, rd, wr)
    assert rel_max(out.cpu().numpy(), o_ref) <= 1e-4
    assert np.array_equal(pool.cpu().numpy(), ref_pool.astype(np.float32))


def test_publish_many_requests():
    R = 1000
    c_np = np.arange(R, dtype=np.int32)
    i_np = np.arange(R, 2 * R, dtype=np.int32)
    c, i = _i32(c_np), _i32(i_np)
    _case("publish R=1000")
    gdn.gdn_publish_slots(c, i)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), i_np) and np.array_equal(i.cpu().numpy(), c_np)
