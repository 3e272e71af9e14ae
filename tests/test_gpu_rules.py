"""GPU parity of the update rules (gated delta, delta, gated, linear) against the
float64 oracle, called through the C ABI: the recurrent kernels (V-major and
K-major, fp32 and fp16 I/O), the chunked prefill, and verify with capsule
followed by replay. Inputs a rule does not read are passed as NULL.

Tolerances as for the gated delta rule: FP32 I/O max|x-y| / max|y| <= 1e-4;
FP16 I/O output max-abs <= 2e-2 and final-state relative L2 <= 1e-3; capsule
decay and key sections 1e-5, deltas 1e-3 (FP16); replay against the GPU's own
recurrence 1e-5.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import cu_from_lengths, make_inputs
from gpu_helpers import (TOL_REPLAY_REL, assert_parity, dev, oracle_forward, rel_max, rule_reads,
                         run_forward)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import gdn_oracle as O                   # noqa: E402
from oracle import layout_oracle as LO               # noqa: E402

RULES = ["gated_delta", "delta", "gated", "linear"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("io,Dk,Dv", [("f32", 64, 32), ("f16", 128, 128), ("f32", 16, 128)])
def test_rule_recurrent_vs_oracle(rule, io, Dk, Dv):
    lengths = [1, 7, 0, 33, 5]
    inp = make_inputs(lengths, 2, 6, Dk, Dv, io, seed=700 + Dk + Dv)
    _case(f"rule {rule} recurrent io={io} Dk={Dk} Dv={Dv} lengths={lengths}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_RECURRENT, rule=rule)
    ref_o, ref_s, _ = oracle_forward(inp, O, rule=rule)
    assert_parity(io, res["output"], ref_o, res["final_state"], ref_s, f"{rule} {io} {Dk}x{Dv}")


@pytest.mark.parametrize("rule", RULES)
def test_rule_chunk_vs_oracle(rule):
    lengths = [1, 63, 64, 65, 130, 0, 200]
    inp = make_inputs(lengths, 2, 4, 128, 128, "f16", seed=710)
    _case(f"rule {rule} chunk lengths={lengths}")
    res = run_forward(inp, torch, gdn, plan=gdn.PLAN_CHUNK, rule=rule)
    ref_o, ref_s, _ = oracle_forward(inp, O, rule=rule)
    assert_parity("f16", res["output"], ref_o, res["final_state"], ref_s, f"{rule} chunk")


@pytest.mark.parametrize("rule", RULES)
def test_rule_capsule_then_replay(rule):
    cap, Hk, Hv, Dk, Dv = 4, 2, 4, 128, 128
    lengths = [4, 4, 3]
    inp = make_inputs(lengths, Hk, Hv, Dk, Dv, "f16", seed=720, capacity=cap)
    _case(f"rule {rule} verify capsule + replay")
    res = run_forward(inp, torch, gdn, capacity=cap, write_final=False, poison=-7.0, rule=rule)
    ref_o, _, ref_cap = oracle_forward(inp, O, capacity=cap, poison=-7.0, rule=rule)
    assert_parity("f16", res["output"], ref_o, what=f"{rule} verify")
    got = res["state_update"]
    sa, sk, sd = O.capsule_sections(Hk, Hv, Dk, Dv)
    assert rel_max(got[..., sa], ref_cap[..., sa]) <= 1e-5
    assert rel_max(got[..., sk], ref_cap[..., sk]) <= 1e-5
    assert rel_max(got[..., sd], ref_cap[..., sd]) <= 1e-3
    assert np.all(got[2, 3:] == -7.0)
    # replay of the accepted prefixes equals the GPU's own recurrence over them
    acc = np.array([4, 2, 0], np.int32)
    s = dev(inp["initial_state"], torch)
    dst = torch.full_like(s, float("nan"))
    gdn.gdn_replay(s, torch.from_numpy(got).cuda(), dev(acc, torch), dst, num_k_heads=Hk,
                   state_update_capacity=cap, accepted_host=acc)
    torch.cuda.synchronize()
    dst = dst.cpu().numpy()
    cu = inp["cu_seqlens"]
    sub = dict(inp)
    idx = np.concatenate([np.arange(cu[r], cu[r] + acc[r]) for r in range(len(acc))]).astype(int)
    for n in ("q", "k", "v", "a", "b"):
        sub[n] = inp[n][idx]
    sub["cu_seqlens"] = cu_from_lengths(acc)
    own = run_forward(sub, torch, gdn, plan=gdn.PLAN_RECURRENT, rule=rule)
    assert rel_max(dst, own["final_state"]) <= TOL_REPLAY_REL
    assert np.array_equal(dst[2], inp["initial_state"][2])


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("plan", ["recurrent", "chunk"])
def test_rule_kmajor_vs_oracle(rule, plan):
    lengths = [5, 70, 1] if plan == "chunk" else [5, 9, 1]
    inp = make_inputs(lengths, 2, 4, 128, 128, "f16", seed=730)
    R = len(lengths)
    M0 = np.random.default_rng(731).standard_normal((R, 4, 128, 128)) * 0.05
    _case(f"rule {rule} K-major {plan}")
    reads_a, reads_b = rule_reads(rule)
    d = {n: dev(inp[n], torch) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens")}
    if not reads_a:
        d["a"] = d["A_log"] = d["dt_bias"] = None
    if not reads_b:
        d["b"] = None
    N = inp["q"].shape[0]
    out = torch.full((N, 4, 128), float("nan"), dtype=torch.float16, device="cuda")
    init = dev(M0.astype(np.float32), torch)
    fin = torch.full_like(init, float("nan"))
    pc = gdn.PLAN_CHUNK if plan == "chunk" else gdn.PLAN_RECURRENT
    nws = gdn.gdn_forward_workspace_bytes(N, R, 2, 4, 128, 128, gdn.GDN_F16, plan=pc,
                                          cu_seqlens_host=inp["cu_seqlens"])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    gdn.gdn_forward(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out,
                    initial_state=init, final_state=fin, cu_seqlens_host=inp["cu_seqlens"], plan=pc,
                    workspace=ws, state_layout=gdn.STATE_K_MAJOR, update_rule=RULES.index(rule))
    torch.cuda.synchronize()
    o_ref, M_ref, _ = LO.gdn_forward_k_major(*[inp[n] for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias",
                                                                 "cu_seqlens")], M0.astype(np.float32),
                                             update_rule=rule)
    assert_parity("f16", out.float().cpu().numpy(), o_ref, fin.cpu().numpy(), M_ref, f"{rule} K-major {plan}")
