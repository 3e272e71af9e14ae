"""GPU parity of the K-major state layout (GDN_STATE_K_MAJOR: states
[.., Dk, Dv]) against the float64 layout oracle, called through the C ABI: the
K-major recurrent kernels (decode, capsule), the chunk path and the replay.

Tolerances as for the V-major calls: FP32 I/O 1e-4 relative; FP16 I/O output
max-abs 2e-2 and state rel-L2 1e-3; replay vs the GPU's own recurrence 1e-5
relative; the capsule (same layout in both state layouts) as in the V-major
capsule tests.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs, workload_inputs
from gpu_helpers import TOL_REPLAY_REL, assert_parity, dev, rel_max

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import gdn_oracle as GO                  # noqa: E402
from oracle import layout_oracle as LO               # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def _args(inp):
    return [inp[n] for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")]


def run_kmajor(inp, M0, *, plan=gdn.PLAN_AUTO, capacity=0, in_place=False, write_final=True):
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    N, Hv, Dv = inp["v"].shape
    R = len(inp["cu_seqlens"]) - 1
    Hk, Dk = inp["Hk"], inp["Dk"]
    init = dev(M0.astype(np.float32), torch) if M0 is not None else None
    fin = None
    if write_final:
        fin = init if in_place else torch.full((R, Hv, Dk, Dv), float("nan"), device="cuda")
    out = torch.full((N, Hv, Dv), float("nan"), dtype=d["v"].dtype, device="cuda")
    su = None
    if capacity:
        su = torch.full((R, capacity, gdn.capsule_width(Hk, Hv, Dk, Dv)), -3.0, device="cuda")
    io = gdn.GDN_F16 if inp["io_dtype"] == "f16" else gdn.GDN_F32
    nws = gdn.gdn_forward_workspace_bytes(N, R, Hk, Hv, Dk, Dv, io, capacity=capacity, plan=plan,
                                          cu_seqlens_host=inp["cu_seqlens"])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                    initial_state=init, final_state=fin, state_update=su, state_update_capacity=capacity,
                    cu_seqlens_host=inp["cu_seqlens"], plan=plan, workspace=ws,
                    state_layout=gdn.STATE_K_MAJOR)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), None if fin is None else fin.cpu().numpy(),
            None if su is None else su.cpu().numpy())


def _m0(inp, seed):
    R = len(inp["cu_seqlens"]) - 1
    return np.random.default_rng(seed).standard_normal((R, inp["Hv"], inp["Dk"], inp["Dv"])) * 0.05


@pytest.mark.parametrize("io", ["f32", "f16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
def test_kmajor_recurrent_shapes(io, Dk, Dv):
    inp = make_inputs([1, 7, 0, 33, 5, 2], 2, 6, Dk, Dv, io, seed=500 + Dk + Dv)
    M0 = _m0(inp, 1)
    _case(f"K-major recurrent {io} Dk={Dk} Dv={Dv}")
    o, M, _ = run_kmajor(inp, M0, plan=gdn.PLAN_RECURRENT)
    o_ref, M_ref, _ = LO.gdn_forward_k_major(*_args(inp), M0.astype(np.float32))
    assert_parity(io, o, o_ref, M, M_ref, f"K-major {io} {Dk}x{Dv}")


def test_kmajor_batched_decode_in_place():
    inp = workload_inputs("batched_decode")
    M0 = LO.to_k_major(inp["initial_state"])
    _case("K-major batched decode fp16 R=64 Hv=32 D=128 in place")
    o, M, _ = run_kmajor(inp, M0, plan=gdn.PLAN_RECURRENT, in_place=True)
    o_ref, M_ref, _ = LO.gdn_forward_k_major(*_args(inp), M0)
    assert_parity("f16", o, o_ref, M, M_ref, "K-major decode")


@pytest.mark.parametrize("Dk,Dv", [(128, 64), (32, 16)])
def test_kmajor_capsule_matches_oracle(Dk, Dv):
    cap = 4
    inp = make_inputs([4, 3, 1, 4], 2, 4, Dk, Dv, "f16", seed=510 + Dv, capacity=cap)
    M0 = _m0(inp, 2)
    _case(f"K-major capsule fp16 capacity 4 Dk={Dk} Dv={Dv}")
    o, M, su = run_kmajor(inp, M0, plan=gdn.PLAN_RECURRENT, capacity=cap)
    init = np.full(su.shape, -3.0)
    o_ref, M_ref, su_ref = LO.gdn_forward_k_major(*_args(inp), M0.astype(np.float32), state_update_capacity=cap,
                                                  state_update_init=init)
    assert_parity("f16", o, o_ref, M, M_ref, "K-major capsule")
    # rows past each request's length keep their poison exactly; the rest match the oracle
    lengths = np.diff(inp["cu_seqlens"])
    for r, n in enumerate(lengths):
        assert np.all(su[r, n:] == -3.0)
    # per section, as for the V-major capsule: decay and unit key are computed
    # from the inputs alone (1e-5); the deltas depend on the state as the outputs
    # do (1e-3 on their scale, FP16 inputs)
    sa, sk, sd = GO.capsule_sections(inp["Hk"], inp["Hv"], Dk, Dv)
    rows = np.concatenate([[(r, j) for j in range(n)] for r, n in enumerate(lengths) if n]).astype(int)
    got, ref = su[rows[:, 0], rows[:, 1]], su_ref[rows[:, 0], rows[:, 1]]
    assert rel_max(got[:, sa], ref[:, sa]) <= 1e-5
    assert rel_max(got[:, sk], ref[:, sk]) <= 1e-5
    assert rel_max(got[:, sd], ref[:, sd]) <= 1e-3


def test_kmajor_chunk_prefill():
    inp = make_inputs([130, 64, 1, 200], 2, 4, 128, 128, "f16", seed=520)
    M0 = _m0(inp, 3)
    _case("K-major chunk prefill fp16")
    o, M, _ = run_kmajor(inp, M0, plan=gdn.PLAN_CHUNK)
    o_ref, M_ref, _ = LO.gdn_forward_k_major(*_args(inp), M0.astype(np.float32))
    assert_parity("f16", o, o_ref, M, M_ref, "K-major chunk")


def test_kmajor_equals_transposed_v_major():
    inp = make_inputs([5, 9, 2], 2, 4, 64, 32, "f32", seed=530)
    M0 = _m0(inp, 4)
    _case("K-major vs V-major on transposed states")
    o_k, M_k, _ = run_kmajor(inp, M0, plan=gdn.PLAN_RECURRENT)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    S0 = dev(np.ascontiguousarray(np.swapaxes(M0, -1, -2)).astype(np.float32), torch)
    fin = torch.empty_like(S0)
    out = torch.empty((16, 4, 32), device="cuda")
    gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                    initial_state=S0, final_state=fin, cu_seqlens_host=inp["cu_seqlens"],
                    plan=gdn.PLAN_RECURRENT)
    torch.cuda.synchronize()
    assert rel_max(o_k, out.cpu().numpy()) <= 1e-5
    assert rel_max(M_k, np.swapaxes(fin.cpu().numpy(), -1, -2)) <= 1e-5


def test_kmajor_replay_vs_own_recurrence():
    T, R, cap = 4, 6, 4
    inp = make_inputs([T] * R, 2, 4, 128, 128, "f16", seed=540, capacity=cap)
    M0 = _m0(inp, 5).astype(np.float32)
    _, _, su = run_kmajor(inp, M0, plan=gdn.PLAN_RECURRENT, capacity=cap, write_final=False)
    acc_np = np.array([0, 1, 2, 3, 4, 2], np.int32)
    src = dev(M0, torch)
    dst = torch.full_like(src, float("nan"))
    _case("K-major replay (params, no slots)")
    gdn.gdn_replay_pooled(src, dev(su, torch), dev(acc_np, torch), dst, num_k_heads=2, state_update_capacity=cap,
                          accepted_host=acc_np, state_layout=gdn.STATE_K_MAJOR, pooled=False)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    ref = LO.gdn_replay_k_major(M0, su, acc_np, 2, 4, 128, 128)
    assert rel_max(got, ref) <= 1e-5
    assert np.array_equal(got[0], M0[0])                     # m = 0 copies the committed state
    for r in range(1, R):
        m, t0 = int(acc_np[r]), int(inp["cu_seqlens"][r])
        sub = {n: inp[n][t0:t0 + m] for n in ("q", "k", "v", "a", "b")}
        sub.update(A_log=inp["A_log"], dt_bias=inp["dt_bias"], cu_seqlens=np.array([0, m], np.int32),
                   Hk=2, Hv=4, Dk=128, Dv=128, io_dtype="f16")
        _, M_gpu, _ = run_kmajor(sub, M0[r:r + 1], plan=gdn.PLAN_RECURRENT)
        assert rel_max(got[r], M_gpu[0]) <= TOL_REPLAY_REL, r


def test_kmajor_pooled_decode():
    R, P = 8, 20
    inp = make_inputs([1] * R, 2, 4, 64, 128, "f16", seed=550)
    rng = np.random.default_rng(6)
    pool = (rng.standard_normal((P, 4, 64, 128)) * 0.05).astype(np.float32)
    perm = rng.permutation(P)
    rd, wr = perm[:R].copy(), perm[R:2 * R].copy()
    rd[2] = -1
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    dpool = dev(pool, torch)
    out = torch.empty((R, 4, 128), dtype=torch.float16, device="cuda")
    _case("K-major pooled decode")
    gdn.gdn_forward_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"],
                           out, num_slots=P, read_slots=dev(rd.astype(np.int32), torch),
                           write_slots=dev(wr.astype(np.int32), torch), read_slots_host=rd, write_slots_host=wr,
                           initial_state=dpool, final_state=dpool, cu_seqlens_host=inp["cu_seqlens"],
                           plan=gdn.PLAN_RECURRENT, state_layout=gdn.STATE_K_MAJOR)
    torch.cuda.synchronize()
    M0 = np.stack([pool[s] if s >= 0 else np.zeros(pool.shape[1:], np.float32) for s in rd])
    o_ref, M_ref, _ = LO.gdn_forward_k_major(*_args(inp), M0)
    got = dpool.cpu().numpy()
    assert_parity("f16", out.float().cpu().numpy(), o_ref, got[wr], M_ref, "K-major pooled")
    untouched = [s for s in range(P) if s not in set(wr)]
    assert np.array_equal(got[untouched], pool[untouched])


def test_kmajor_pooled_replay():
    T, R, cap, P = 4, 5, 4, 12
    inp = make_inputs([T] * R, 2, 4, 64, 32, "f32", seed=560, capacity=cap)
    rng = np.random.default_rng(8)
    pool = (rng.standard_normal((P, 4, 64, 32)) * 0.05).astype(np.float32)
    perm = rng.permutation(P)
    rd, wr = perm[:R].copy(), perm[R:2 * R].copy()
    _, _, su = run_kmajor(inp, pool[rd], plan=gdn.PLAN_RECURRENT, capacity=cap, write_final=False)
    acc_np = np.array([0, 4, 1, 3, 2], np.int32)
    dpool = dev(pool, torch)
    _case("K-major pooled replay")
    gdn.gdn_replay_pooled(dpool, dev(su, torch), dev(acc_np, torch), dpool, num_k_heads=2,
                          state_update_capacity=cap, read_slots=dev(rd.astype(np.int32), torch),
                          write_slots=dev(wr.astype(np.int32), torch), read_slots_host=rd, write_slots_host=wr,
                          accepted_host=acc_np, state_layout=gdn.STATE_K_MAJOR)
    torch.cuda.synchronize()
    got = dpool.cpu().numpy()
    ref = LO.gdn_replay_k_major(pool[rd], su, acc_np, 2, 4, 64, 32)
    assert rel_max(got[wr], ref) <= 1e-5
    untouched = [s for s in range(P) if s not in set(wr)]
    assert np.array_equal(got[untouched], pool[untouched])
