"""GPU parity of the causal convolution fused into the GatedDeltaNet decode
(gdn_conv_decode_forward), called through the C ABI.

The fused call must equal the two separate calls it replaces, bit for bit:
gdn_conv_forward over the concatenated [q | k | v] channels, then gdn_forward
(token-recurrent plan) on the split output. It rounds the convolution's output
to the I/O type exactly as the stored output of gdn_conv_forward is rounded, and
runs the same recurrence code, so output, final state and the convolution's new
carried inputs compare with ==. Against the float64 oracles (the convolution,
then the recurrence on its output) the tolerances are the operator's: FP16 I/O
output max-abs <= 2e-2 and final-state relative L2 <= 1e-3, FP32 I/O 1e-4
relative; the carried inputs are copies of inputs and compare exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs
from gdn_workloads.conv import conv_channels, make_conv_inputs
from gpu_helpers import RULE_NAMES, assert_parity, dev, rule_reads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import conv_oracle as CO                 # noqa: E402
from oracle import gdn_oracle as O                   # noqa: E402

K = 4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()                                         # fails loudly if libgdn.so is missing


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def _inputs(lengths, Hk, Hv, D, io, seed, *, gdn_initial="normal", conv_initial="normal"):
    g = make_inputs(lengths, Hk, Hv, D, D, io, seed, initial=gdn_initial)
    c = make_conv_inputs(lengths, conv_channels(Hk, Hv, D, D), K, io, seed + 1, initial=conv_initial)
    return g, c


def _device(g, c, rule, bias):
    d = {n: (dev(g[n], torch) if g[n] is not None else None)
         for n in ("a", "b", "A_log", "dt_bias", "cu_seqlens", "initial_state")}
    reads_a, reads_b = rule_reads(rule)
    if not reads_a:
        d["a"] = d["A_log"] = d["dt_bias"] = None
    if not reads_b:
        d["b"] = None
    d["mixed"] = dev(c["x"], torch)
    d["weight"] = dev(c["weight"], torch)
    d["bias"] = dev(c["bias"], torch) if bias else None
    d["conv_init"] = dev(c["initial_state"], torch) if c["initial_state"] is not None else None
    return d


def run_separate(g, c, *, rule="gated_delta", act=gdn.CONV_SILU, bias=True, dense=False):
    """gdn_conv_forward over all channels, then gdn_forward on the split output."""
    d = _device(g, c, rule, bias)
    Hk, Hv, D = g["Hk"], g["Hv"], g["Dk"]
    N, Cm = c["x"].shape
    R = len(g["lengths"])
    io = d["mixed"].dtype
    y = torch.empty((N, Cm), dtype=io, device="cuda")
    cfin = torch.full((R, Cm, K - 1), float("nan"), device="cuda")
    cu = None if dense else d["cu_seqlens"]
    cu_host = None if dense else g["cu_seqlens"]
    gdn.gdn_conv_forward(d["mixed"], d["weight"], d["bias"], cu, y, initial_state=d["conv_init"],
                         final_state=cfin, cu_seqlens_host=cu_host, activation=act,
                         num_reqs=R if dense else None)
    q = y[:, :Hk * D].reshape(N, Hk, D).contiguous()
    k = y[:, Hk * D:2 * Hk * D].reshape(N, Hk, D).contiguous()
    v = y[:, 2 * Hk * D:].reshape(N, Hv, D).contiguous()
    out = torch.full((N, Hv, D), float("nan"), dtype=io, device="cuda")
    fin = torch.full((R, Hv, D, D), float("nan"), device="cuda")
    gdn.gdn_forward(q, k, v, d["a"], d["b"], d["A_log"], d["dt_bias"], cu, out,
                    initial_state=d["initial_state"], final_state=fin, cu_seqlens_host=cu_host,
                    plan=gdn.PLAN_RECURRENT, update_rule=RULE_NAMES.index(rule),
                    num_reqs=R if dense else None)
    torch.cuda.synchronize()
    return {"output": out.cpu(), "final_state": fin.cpu(), "conv_final": cfin.cpu(), "y": y.cpu()}


def run_fused(g, c, *, rule="gated_delta", act=gdn.CONV_SILU, bias=True, dense=False, write_conv=True,
              write_final=True):
    d = _device(g, c, rule, bias)
    Hk, Hv, D = g["Hk"], g["Hv"], g["Dk"]
    N, Cm = c["x"].shape
    R = len(g["lengths"])
    io = d["mixed"].dtype
    out = torch.full((N, Hv, D), float("nan"), dtype=io, device="cuda")
    fin = torch.full((R, Hv, D, D), float("nan"), device="cuda") if write_final else None
    cfin = torch.full((R, Cm, K - 1), float("nan"), device="cuda") if write_conv else None
    gdn.gdn_conv_decode_forward(d["mixed"], d["weight"], d["bias"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                None if dense else d["cu_seqlens"], out, num_k_heads=Hk, head_k_dim=D,
                                conv_initial_state=d["conv_init"], conv_final_state=cfin, conv_activation=act,
                                initial_state=d["initial_state"], final_state=fin,
                                cu_seqlens_host=None if dense else g["cu_seqlens"],
                                update_rule=RULE_NAMES.index(rule), num_reqs=R if dense else None)
    torch.cuda.synchronize()
    return {"output": out.cpu(), "final_state": None if fin is None else fin.cpu(),
            "conv_final": None if cfin is None else cfin.cpu()}


def _bitwise(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), what


def _check_equal(fu, se, what):
    _bitwise(fu["output"], se["output"], f"{what}: output")
    if fu["final_state"] is not None:
        _bitwise(fu["final_state"], se["final_state"], f"{what}: final state")
    if fu["conv_final"] is not None:
        _bitwise(fu["conv_final"], se["conv_final"], f"{what}: carried inputs")


CASES = [
    # lengths, Hk, Hv, D, io
    ([1] * 64, 16, 32, 128, "f16"),                 # the batched decode step
    ([1, 0, 2, 3, 5, 9, 1], 2, 4, 128, "f16"),      # segments shorter and longer than K - 1, an empty one
    ([1, 0, 2, 3, 5, 9, 1], 2, 4, 128, "f32"),
    ([3, 1, 4], 2, 4, 64, "f16"),
    ([3, 1, 4], 1, 3, 32, "f32"),
    ([2, 7], 2, 2, 16, "f16"),
]


@pytest.mark.parametrize("lengths,Hk,Hv,D,io", CASES)
def test_fused_equals_separate(lengths, Hk, Hv, D, io):
    g, c = _inputs(lengths, Hk, Hv, D, io, seed=1200 + D + len(lengths))
    _case(f"conv decode fused vs separate lengths={lengths[:8]} Hk={Hk} Hv={Hv} D={D} {io}")
    _check_equal(run_fused(g, c), run_separate(g, c), "fused = separate")


@pytest.mark.parametrize("rule", ["delta", "gated", "linear"])
def test_fused_equals_separate_rules(rule):
    g, c = _inputs([2, 1, 4], 2, 4, 128, "f16", seed=1300)
    _case(f"conv decode fused vs separate rule={rule}")
    _check_equal(run_fused(g, c, rule=rule), run_separate(g, c, rule=rule), f"rule {rule}")


def test_fused_equals_separate_optional_inputs():
    # no carried inputs, no bias, no activation, no initial state; then no outputs of state
    g, c = _inputs([1, 3, 0, 2], 2, 4, 128, "f16", seed=1310, gdn_initial="zero", conv_initial="zero")
    _case("conv decode: zero states, no bias, identity activation")
    kw = dict(act=gdn.CONV_NONE, bias=False)
    _check_equal(run_fused(g, c, **kw), run_separate(g, c, **kw), "optional inputs")
    fu = run_fused(g, c, write_conv=False, write_final=False)
    _bitwise(fu["output"], run_separate(g, c)["output"], "outputs only")


def test_fused_dense_layout():
    g, c = _inputs([2, 2, 2], 2, 4, 128, "f16", seed=1320)
    _case("conv decode dense layout")
    _check_equal(run_fused(g, c, dense=True), run_separate(g, c), "dense = packed")


def test_fused_no_tokens_copies_the_states():
    g, c = _inputs([0, 0, 0], 2, 4, 128, "f16", seed=1330)
    _case("conv decode, requests without tokens")
    fu = run_fused(g, c)
    assert np.array_equal(fu["final_state"].numpy(), g["initial_state"])
    assert np.array_equal(fu["conv_final"].numpy(), c["initial_state"])


def _oracle(g, c, *, act="silu"):
    y, cfin, _ = CO.conv_forward(c["x"], c["weight"], c["bias"], g["cu_seqlens"], c["initial_state"],
                                 activation=act)
    Hk, Hv, D = g["Hk"], g["Hv"], g["Dk"]
    N = y.shape[0]
    q = y[:, :Hk * D].reshape(N, Hk, D)
    k = y[:, Hk * D:2 * Hk * D].reshape(N, Hk, D)
    v = y[:, 2 * Hk * D:].reshape(N, Hv, D)
    o, fin, _ = O.gdn_forward(q, k, v, g["a"], g["b"], g["A_log"], g["dt_bias"], g["cu_seqlens"],
                              g["initial_state"])
    return o, fin, cfin


@pytest.mark.parametrize("io", ["f16", "f32"])
def test_fused_vs_oracle(io):
    g, c = _inputs([1, 0, 2, 3, 5, 1], 2, 4, 128, io, seed=1340)
    _case(f"conv decode vs oracle {io}")
    fu = run_fused(g, c)
    o, fin, cfin = _oracle(g, c)
    assert_parity(io, fu["output"].float().numpy(), o, fu["final_state"].numpy(), fin, "conv decode")
    assert np.array_equal(fu["conv_final"].numpy(), cfin.astype(np.float32))


def test_two_chained_decode_steps():
    # step 2 reads the banks step 1 wrote; both steps equal the separate calls
    g1, c1 = _inputs([1] * 8, 2, 4, 128, "f16", seed=1350)
    g2, c2 = _inputs([1] * 8, 2, 4, 128, "f16", seed=1351)
    _case("conv decode two chained steps")
    s1 = run_fused(g1, c1)
    g2["initial_state"] = s1["final_state"].numpy()
    c2["initial_state"] = s1["conv_final"].numpy()
    _check_equal(run_fused(g2, c2), run_separate(g2, c2), "second step")
