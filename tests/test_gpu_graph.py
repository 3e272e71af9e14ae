"""GPU: the hot path captured in HIP graphs (torch.cuda.CUDAGraph) and replayed.

A serving loop captures a decode step (also with the causal convolution fused
in), or the speculative step (verify, replay of the accepted prefix, publication
of the slot arrays; or the fused step and the publication), once and replays it.
Each graph here is replayed several times, with the program's own eager work
and synchronisations between the replays, and every replay is compared bit for
bit with the same calls made eagerly from the same starting state (the kernels
are deterministic: no atomics, fixed reduction order). The calls are given host
mirrors of cu_seqlens, so nothing in them waits for the device. The last test
runs two independent calls on two streams at once.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs
from gdn_workloads.conv import make_conv_inputs
from gpu_helpers import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()                                         # fails loudly if libgdn.so is missing


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _snapshot(tensors):
    torch.cuda.synchronize()
    return [t.detach().cpu().clone() for t in tensors]


def _same(got, ref, what):
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), f"{what}: tensor {i} differs"


def test_decode_steps_graph():
    # three in-place decode steps per replay over one state bank
    R, Hk, Hv, D, steps = 8, 4, 8, 128, 3
    inp = make_inputs([1] * R, Hk, Hv, D, D, "f16", seed=501)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    s0 = dev(inp["initial_state"], torch)
    state = s0.clone()
    out = torch.empty((R, Hv, D), dtype=torch.float16, device="cuda")

    def run():
        for _ in range(steps):
            gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"],
                            out, initial_state=state, final_state=state, cu_seqlens_host=inp["cu_seqlens"],
                            plan=gdn.PLAN_RECURRENT)

    _case("decode: eager reference")
    run()
    ref = _snapshot([state, out])
    _case("decode: capture")
    g = _capture(run)
    for rep in range(3):
        state.copy_(s0)
        out.zero_()
        torch.cuda.synchronize()
        _case(f"decode: replay {rep}")
        g.replay()
        _same(_snapshot([state, out]), ref, f"decode replay {rep}")


def test_speculative_step_graph_publishes_on_the_device():
    # verify from the committed slots, replay the accepted prefix into the
    # inactive ones, swap the slot arrays: replay k of the graph must equal k
    # eager steps, since each replay reads the slots the previous one published
    T, R, cap, Hk, Hv, D = 4, 6, 4, 2, 4, 128
    inp = make_inputs([T] * R, Hk, Hv, D, D, "f16", seed=502, capacity=cap)
    P = 2 * R
    rng = np.random.default_rng(7)
    perm = rng.permutation(P)
    committed_np, inactive_np = perm[:R], perm[R:]
    pool_np = rng.standard_normal((P, Hv, D, D)).astype(np.float32) * 0.05
    pool_np[committed_np] = inp["initial_state"]
    accepted = _i32([0, 1, 2, 3, 4, 2])
    pool0 = dev(pool_np, torch)
    pool = pool0.clone()
    committed, inactive = _i32(committed_np), _i32(inactive_np)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    out = torch.empty((T * R, Hv, D), dtype=torch.float16, device="cuda")
    su = torch.zeros((R, cap, gdn.capsule_width(Hk, Hv, D, D)), device="cuda")

    def step():
        gdn.gdn_forward_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                               d["cu_seqlens"], out, num_slots=P, read_slots=committed, write_slots=None,
                               initial_state=pool, final_state=None, state_update=su,
                               state_update_capacity=cap, cu_seqlens_host=inp["cu_seqlens"],
                               plan=gdn.PLAN_RECURRENT)
        gdn.gdn_replay_pooled(pool, su, accepted, pool, num_k_heads=Hk, state_update_capacity=cap,
                              read_slots=committed, write_slots=inactive)
        gdn.gdn_publish_slots(committed, inactive)

    def reset():
        pool.copy_(pool0)
        committed.copy_(_i32(committed_np))
        inactive.copy_(_i32(inactive_np))
        out.zero_()
        su.zero_()
        torch.cuda.synchronize()

    watched = [pool, committed, inactive, out, su]
    _case("speculative step: eager reference, 3 steps")
    refs = []
    for _ in range(3):
        step()
        refs.append(_snapshot(watched))
    reset()
    _case("speculative step: capture")
    g = _capture(step)
    for trial in range(2):
        reset()
        for k in range(3):
            _case(f"speculative step: trial {trial} replay {k}")
            g.replay()
            _same(_snapshot(watched), refs[k], f"trial {trial} replay {k}")


def test_fused_speculative_step_graph():
    # the fused step over the pool (replay of the previous capsule's accepted
    # prefix from the committed slots into the inactive ones, verify from that
    # state) and the publication; two steps per graph, since the capsule buffers
    # alternate: replay k of the graph must equal 2 (k + 1) eager steps
    T, R, cap, Hk, Hv, D = 4, 6, 4, 2, 4, 128
    inp = make_inputs([T] * R, Hk, Hv, D, D, "f16", seed=503, capacity=cap)
    P = 2 * R
    rng = np.random.default_rng(8)
    perm = rng.permutation(P)
    committed_np, inactive_np = perm[:R], perm[R:]
    pool_np = rng.standard_normal((P, Hv, D, D)).astype(np.float32) * 0.05
    pool_np[committed_np] = inp["initial_state"]
    accepted = _i32([0, 1, 2, 3, 4, 2])
    accepted_host = np.array([0, 1, 2, 3, 4, 2], np.int32)
    pool0 = dev(pool_np, torch)
    pool = pool0.clone()
    committed, inactive = _i32(committed_np), _i32(inactive_np)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    out = torch.empty((T * R, Hv, D), dtype=torch.float16, device="cuda")
    W = gdn.capsule_width(Hk, Hv, D, D)
    caps0 = [torch.randn((R, cap, W), device="cuda") * 0.01 for _ in range(2)]
    caps = [c.clone() for c in caps0]

    def one(k):
        gdn.gdn_replay_forward_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                      d["cu_seqlens"], out, num_slots=P, read_slots=committed,
                                      write_slots=inactive, initial_state=pool, replay_pool=pool,
                                      prev_state_update=caps[(k + 1) % 2], state_update=caps[k % 2],
                                      state_update_capacity=cap, accepted=accepted, accepted_host=accepted_host,
                                      cu_seqlens_host=inp["cu_seqlens"], plan=gdn.PLAN_RECURRENT)
        gdn.gdn_publish_slots(committed, inactive)

    def two():
        one(0)
        one(1)

    def reset():
        pool.copy_(pool0)
        committed.copy_(_i32(committed_np))
        inactive.copy_(_i32(inactive_np))
        for c, c0 in zip(caps, caps0):
            c.copy_(c0)
        out.zero_()
        torch.cuda.synchronize()

    watched = [pool, committed, inactive, out, caps[0], caps[1]]
    _case("fused speculative step: eager reference, 3 x 2 steps")
    refs = []
    for _ in range(3):
        two()
        refs.append(_snapshot(watched))
    reset()
    _case("fused speculative step: capture")
    g = _capture(two)
    for trial in range(2):
        reset()
        for k in range(3):
            _case(f"fused speculative step: trial {trial} replay {k}")
            g.replay()
            _same(_snapshot(watched), refs[k], f"fused trial {trial} replay {k}")


def test_chunked_prefill_graph():
    lengths = [130, 64, 1, 77]
    Hk, Hv, D = 2, 4, 128
    inp = make_inputs(lengths, Hk, Hv, D, D, "f16", seed=503)
    N, R = sum(lengths), len(lengths)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    init = dev(inp["initial_state"], torch)
    fin = torch.empty_like(init)
    out = torch.empty((N, Hv, D), dtype=torch.float16, device="cuda")
    nws = gdn.gdn_forward_workspace_bytes(N, R, Hk, Hv, D, D, gdn.GDN_F16, cu_seqlens_host=inp["cu_seqlens"])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def run():
        gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                        initial_state=init, final_state=fin, cu_seqlens_host=inp["cu_seqlens"], workspace=ws,
                        plan=gdn.PLAN_CHUNK)

    _case("chunked prefill: eager reference")
    run()
    ref = _snapshot([fin, out])
    _case("chunked prefill: capture")
    g = _capture(run)
    for rep in range(3):
        fin.zero_()
        out.zero_()
        ws.zero_()                                     # the workspace carries nothing between calls
        torch.cuda.synchronize()
        _case(f"chunked prefill: replay {rep}")
        g.replay()
        _same(_snapshot([fin, out]), ref, f"chunked prefill replay {rep}")


def test_conv_decode_graph():
    R, C, K, steps = 16, 2048, 4, 3
    inp = make_conv_inputs([1] * R, C, K, "f16", seed=504)
    x = dev(inp["x"], torch)
    w, b, cu = dev(inp["weight"], torch), dev(inp["bias"], torch), dev(inp["cu_seqlens"], torch)
    s0 = dev(inp["initial_state"], torch)
    state = s0.clone()
    out = torch.empty_like(x)

    def run():
        for _ in range(steps):
            gdn.gdn_conv_forward(x, w, b, cu, out, initial_state=state, final_state=state,
                                 cu_seqlens_host=inp["cu_seqlens"])

    _case("conv decode: eager reference")
    run()
    ref = _snapshot([state, out])
    _case("conv decode: capture")
    g = _capture(run)
    for rep in range(3):
        state.copy_(s0)
        out.zero_()
        torch.cuda.synchronize()
        _case(f"conv decode: replay {rep}")
        g.replay()
        _same(_snapshot([state, out]), ref, f"conv decode replay {rep}")


def test_conv_fused_decode_graph():
    # three decode steps with the convolution fused: the GDN state in place, the
    # carried inputs passed from bank to bank (A -> B -> A -> B)
    R, Hk, Hv, D, K = 8, 2, 4, 128, 4
    C = 2 * Hk * D + Hv * D
    g_in = make_inputs([1] * R, Hk, Hv, D, D, "f16", seed=505)
    c_in = make_conv_inputs([1] * R, C, K, "f16", seed=506)
    d = {n: dev(g_in[n], torch) for n in ("a", "b", "A_log", "dt_bias", "cu_seqlens")}
    x, w, b = dev(c_in["x"], torch), dev(c_in["weight"], torch), dev(c_in["bias"], torch)
    s0, c0 = dev(g_in["initial_state"], torch), dev(c_in["initial_state"], torch)
    state, ca, cb = s0.clone(), c0.clone(), torch.zeros_like(c0)
    out = torch.empty((R, Hv, D), dtype=torch.float16, device="cuda")

    def run():
        for src, dst in ((ca, cb), (cb, ca), (ca, cb)):
            gdn.gdn_conv_decode_forward(x, w, b, d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                                        num_k_heads=Hk, head_k_dim=D, conv_initial_state=src,
                                        conv_final_state=dst, initial_state=state, final_state=state,
                                        cu_seqlens_host=g_in["cu_seqlens"])

    def reset():
        state.copy_(s0)
        ca.copy_(c0)
        cb.zero_()
        out.zero_()
        torch.cuda.synchronize()

    _case("fused conv decode: eager reference")
    run()
    ref = _snapshot([state, ca, cb, out])
    reset()
    _case("fused conv decode: capture")
    g = _capture(run)
    for rep in range(3):
        reset()
        _case(f"fused conv decode: replay {rep}")
        g.replay()
        _same(_snapshot([state, ca, cb, out]), ref, f"fused conv decode replay {rep}")


def test_two_streams_run_independent_calls():
    # the library keeps no state between calls: a decode on one stream and a
    # chunked prefill on another, in flight together, each equal their calls made
    # alone (bit for bit)
    dec = make_inputs([1] * 16, 4, 8, 128, 128, "f16", seed=505)
    pre = make_inputs([200, 33], 2, 4, 128, 128, "f16", seed=506)
    dd = {n: dev(dec[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    pd = {n: dev(pre[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    s_dec0 = dev(dec["initial_state"], torch)
    s_dec = s_dec0.clone()
    o_dec = torch.empty((16, 8, 128), dtype=torch.float16, device="cuda")
    init = dev(pre["initial_state"], torch)
    fin = torch.empty_like(init)
    o_pre = torch.empty((233, 4, 128), dtype=torch.float16, device="cuda")
    nws = gdn.gdn_forward_workspace_bytes(233, 2, 2, 4, 128, 128, gdn.GDN_F16, cu_seqlens_host=pre["cu_seqlens"])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def decode_steps(stream):
        for _ in range(4):
            gdn.gdn_forward(dd["q"], dd["k"], dd["v"], dd["a"], dd["b"], dd["A_log"], dd["dt_bias"],
                            dd["cu_seqlens"], o_dec, initial_state=s_dec, final_state=s_dec,
                            cu_seqlens_host=dec["cu_seqlens"], plan=gdn.PLAN_RECURRENT, stream=stream)

    def prefill(stream):
        gdn.gdn_forward(pd["q"], pd["k"], pd["v"], pd["a"], pd["b"], pd["A_log"], pd["dt_bias"], pd["cu_seqlens"],
                        o_pre, initial_state=init, final_state=fin, cu_seqlens_host=pre["cu_seqlens"],
                        workspace=ws, plan=gdn.PLAN_CHUNK, stream=stream)

    _case("two streams: each call alone")
    decode_steps(None)
    prefill(None)
    ref = _snapshot([s_dec, o_dec, fin, o_pre])
    s_dec.copy_(s_dec0)
    fin.zero_()
    o_pre.zero_()
    torch.cuda.synchronize()
    _case("two streams: together")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()      # default priority
    with torch.cuda.stream(sa):
        decode_steps(sa)
    with torch.cuda.stream(sb):
        prefill(sb)
    torch.cuda.synchronize()
    _same(_snapshot([s_dec, o_dec, fin, o_pre]), ref, "two streams")
