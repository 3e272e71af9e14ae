"""GPU parity of the compact causal convolution (gdn_conv_forward,
gdn_conv_replay) against the float64 oracle, called through the C ABI.

Tolerances:
  FP32 I/O  output max|x-y| / max|y| <= 1e-4
  FP16 I/O  output max-abs <= 2e-2
  final state, capture rows and replayed state: bit-exact (they are copies of
  inputs), and capture rows that are not written keep their poison.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads.conv import conv_channels, make_conv_inputs
from gpu_helpers import TOL_F16_OUT_ABS, TOL_F32_REL, dev, max_abs, rel_max

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402
from oracle import conv_oracle as CO                 # noqa: E402

POISON = np.float32(-7.75)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()                                         # fails loudly if libgdn.so is missing


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def run_conv(inp, *, activation="silu", bias=True, initial=True, write_final=True, in_place=False,
             capture=False, counts=False, dense=False, host_cu=True):
    """One gdn_conv_forward call on fresh device copies; returns numpy results."""
    x, C, K = inp["x"], inp["C"], inp["K"]
    N = x.shape[0]
    R = len(inp["lengths"])
    io = torch.float16 if inp["io_dtype"] == "f16" else torch.float32
    dx = dev(x, torch)
    out = torch.full((N, C), float("nan"), dtype=io, device="cuda")
    init = dev(inp["initial_state"], torch) if initial and inp["initial_state"] is not None else None
    fin = None
    if write_final:
        fin = init if in_place else torch.full((R, C, K - 1), float("nan"), device="cuda")
    cap = inp["capacity"] if capture else 0
    su = torch.full((R, cap, C), float(POISON), device="cuda") if capture else None
    cc = dev(inp["capture_count"], torch) if counts else None
    cu = None if dense else dev(inp["cu_seqlens"], torch)
    gdn.gdn_conv_forward(dx, dev(inp["weight"], torch), dev(inp["bias"], torch) if bias else None,
                         cu, out, initial_state=init, final_state=fin, state_update=su,
                         capture_count=cc,
                         cu_seqlens_host=inp["cu_seqlens"] if (host_cu and not dense) else None,
                         activation=gdn.CONV_SILU if activation == "silu" else gdn.CONV_NONE,
                         state_update_capacity=cap, num_reqs=R if dense else None)
    torch.cuda.synchronize()
    return {"output": out.float().cpu().numpy(),
            "final_state": None if fin is None else fin.cpu().numpy(),
            "state_update": None if su is None else su.cpu().numpy()}


def run_oracle(inp, *, activation="silu", bias=True, initial=True, capture=False, counts=False,
               channels=None):
    """The oracle on every channel, or on the listed ones only (the convolution
    is depthwise, so a channel's results depend on that channel alone)."""
    ch = slice(None) if channels is None else np.asarray(channels)
    cap = inp["capacity"] if capture else 0
    init = None
    if capture:
        C = inp["C"] if channels is None else len(channels)
        init = np.full((len(inp["lengths"]), cap, C), POISON, np.float64)
    state = inp["initial_state"][:, ch] if initial and inp["initial_state"] is not None else None
    return CO.conv_forward(inp["x"][:, ch], inp["weight"][ch], inp["bias"][ch] if bias else None,
                           inp["cu_seqlens"], state, activation=activation,
                           state_update_capacity=cap,
                           capture_count=inp["capture_count"] if counts else None,
                           state_update_init=init)


def sample_channels(C, n=256, seed=0):
    """Channels the oracle checks at full width: the first and last 32 and a random
    spread in between (every workgroup's channel group is touched)."""
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(32, C - 32), size=min(n, C - 64), replace=False)
    return np.unique(np.concatenate([np.arange(32), mid, np.arange(C - 32, C)]))


def restrict(res, channels):
    out = dict(res)
    out["output"] = res["output"][:, channels]
    if res["final_state"] is not None:
        out["final_state"] = res["final_state"][:, channels]
    if res["state_update"] is not None:
        out["state_update"] = res["state_update"][:, :, channels]
    return out


def check(inp, res, ref, what=""):
    out, fin, cap = ref
    if inp["io_dtype"] == "f32":
        err = rel_max(res["output"], out)
        assert err <= TOL_F32_REL, f"{what}: output rel-max {err:.3e}"
    else:
        err = max_abs(res["output"], out)
        assert err <= TOL_F16_OUT_ABS, f"{what}: output max-abs {err:.3e}"
    if res["final_state"] is not None:
        assert np.array_equal(res["final_state"], fin.astype(np.float32)), f"{what}: final state"
    if res["state_update"] is not None:
        assert np.array_equal(res["state_update"], cap.astype(np.float32)), f"{what}: capture"


LENGTHS = [1, 7, 0, 33, 5, 64, 2, 130, 3]


@pytest.mark.parametrize("io", ["f32", "f16"])
@pytest.mark.parametrize("K", [2, 3, 4, 5, 8])
def test_ragged_kernel_sizes(io, K):
    # C = 1100 spans two channel groups of 1024 with a ragged second one
    inp = make_conv_inputs(LENGTHS, 1100, K, io, seed=200 + K)
    _case(f"conv ragged {io} K={K} C=1100 lengths={LENGTHS}")
    check(inp, run_conv(inp), run_oracle(inp), f"{io} K={K}")


@pytest.mark.parametrize("io,in_place", [("f32", False), ("f16", False), ("f16", True)])
def test_long_blocks_cross_requests(io, in_place):
    # enough tokens that each workgroup walks many tokens and crosses request
    # boundaries, with empty and shorter-than-window requests in between
    rng = np.random.default_rng(7)
    lengths = list(rng.integers(0, 3000, 40))
    lengths[3] = 0
    lengths[10] = 1
    lengths[11] = 2
    lengths[25] = 0
    inp = make_conv_inputs(lengths, 1028, 4, io, seed=210)
    _case(f"conv long ragged {io} N={sum(lengths)} C=1028 K=4 in_place={in_place}")
    ch = sample_channels(1028, 64)
    check(inp, restrict(run_conv(inp, in_place=in_place), ch), run_oracle(inp, channels=ch), io)


def test_variants_no_bias_no_state_identity():
    inp = make_conv_inputs(LENGTHS, 256, 4, "f32", seed=220)
    _case("conv f32 no bias, zero state, identity activation")
    res = run_conv(inp, activation="none", bias=False, initial=False)
    check(inp, res, run_oracle(inp, activation="none", bias=False, initial=False), "variants")


def test_in_place_final_state():
    inp = make_conv_inputs(LENGTHS, 512, 4, "f16", seed=230)
    _case("conv f16 in place final_state == initial_state")
    check(inp, run_conv(inp, in_place=True), run_oracle(inp), "in place")


def test_without_final_state():
    inp = make_conv_inputs(LENGTHS, 64, 3, "f32", seed=231)
    _case("conv f32 final_state NULL")
    res = run_conv(inp, write_final=False)
    assert res["final_state"] is None
    check(inp, res, run_oracle(inp), "no final")


@pytest.mark.parametrize("counts", [False, True])
def test_capture_rows(counts):
    inp = make_conv_inputs([4, 1, 0, 6, 3, 4, 2], 1100, 4, "f16", seed=240, capacity=4,
                           draw_counts=True)
    _case(f"conv f16 capture capacity 4 counts={counts}")
    res = run_conv(inp, capture=True, counts=counts)
    check(inp, res, run_oracle(inp, capture=True, counts=counts), f"capture counts={counts}")


def test_dense_layout_matches_packed():
    inp = make_conv_inputs([5] * 12, 2048, 4, "f16", seed=250, capacity=3)
    _case("conv f16 dense [12, 5, 2048] vs packed")
    dense = run_conv(inp, dense=True, capture=True)
    packed = run_conv(inp, capture=True)
    for k in ("output", "final_state", "state_update"):
        assert np.array_equal(dense[k], packed[k]), k
    check(inp, dense, run_oracle(inp, capture=True), "dense")


def test_no_tokens_copies_state():
    inp = make_conv_inputs([0, 0, 0], 128, 4, "f32", seed=260)
    _case("conv N=0 R=3: final state is the initial state")
    res = run_conv(inp)
    assert np.array_equal(res["final_state"], inp["initial_state"])


def test_without_host_mirror():
    inp = make_conv_inputs(LENGTHS, 1100, 4, "f16", seed=270)
    _case("conv f16 without cu_seqlens_host")
    check(inp, run_conv(inp, host_cu=False), run_oracle(inp), "no host cu")


def test_uniform_lengths_with_and_without_mirror():
    # equal lengths with a host mirror take the dense indexing; without one, the search
    inp = make_conv_inputs([3] * 40, 1100, 4, "f16", seed=275, capacity=2)
    _case("conv f16 40 x 3 tokens, host mirror vs none")
    a = run_conv(inp, capture=True)
    b = run_conv(inp, capture=True, host_cu=False)
    for k in ("output", "final_state", "state_update"):
        assert np.array_equal(a[k], b[k]), k
    check(inp, a, run_oracle(inp, capture=True), "uniform")


@pytest.mark.parametrize("R,S", [(64, 1), (16, 4)])
def test_decode_and_verify_full_width(R, S):
    C = conv_channels(16, 48, 128, 128)
    inp = make_conv_inputs([S] * R, C, 4, "f16", seed=280 + S, capacity=S, draw_counts=True)
    _case(f"conv f16 {R} x {S} tokens C={C} capture")
    res = run_conv(inp, capture=True, counts=True, in_place=True)
    check(inp, res, run_oracle(inp, capture=True, counts=True), f"{R}x{S}")


def test_ragged_prefill_full_size():
    C = conv_channels(16, 32, 128, 128)
    inp = make_conv_inputs(None, C, 4, "f16", seed=3, num_drawn=8, max_drawn=4096)
    N = int(inp["lengths"].sum())
    _case(f"conv f16 ragged prefill N={N} C={C}")
    ch = sample_channels(C)
    check(inp, restrict(run_conv(inp), ch), run_oracle(inp, channels=ch), "ragged prefill")


# ------------------------------------------------------------------ replay
def _replay(src, su, accepted, cap, accepted_host=True):
    dst = torch.full_like(src, float("nan"))
    gdn.gdn_conv_replay(src, su, accepted, dst, state_update_capacity=cap,
                        accepted_host=accepted.cpu().numpy() if accepted_host else None)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


@pytest.mark.parametrize("K", [2, 4, 8])
def test_replay_matches_oracle_and_prefix_forward(K):
    cap = 6
    R = 9
    inp = make_conv_inputs([cap] * R, 1100, K, "f32", seed=300 + K, capacity=cap,
                           draw_accepted=True)
    inp["accepted"][:3] = [0, cap, 1]
    _case(f"conv replay K={K} cap={cap} accepted={list(inp['accepted'])}")
    res = run_conv(inp, capture=True)
    src = dev(inp["initial_state"], torch)
    su = dev(res["state_update"], torch)
    acc = dev(inp["accepted"], torch)
    got = _replay(src, su, acc, cap)
    ref = CO.conv_replay(inp["initial_state"], res["state_update"], inp["accepted"])
    assert np.array_equal(got, ref.astype(np.float32))
    # the replayed state is the final state of a forward over the accepted prefix
    for r in range(R):
        m = int(inp["accepted"][r])
        t0 = int(inp["cu_seqlens"][r])
        _, fin, _ = CO.conv_forward(inp["x"][t0:t0 + m], inp["weight"], inp["bias"], [0, m],
                                    inp["initial_state"][r:r + 1])
        assert np.array_equal(got[r], fin[0].astype(np.float32)), r
    # device values outside [0, capacity] are clamped
    acc_bad = torch.tensor([-3] + [cap + 5] * (R - 1), dtype=torch.int32, device="cuda")
    got = _replay(src, su, acc_bad, cap, accepted_host=False)
    clamped = np.array([0] + [cap] * (R - 1), np.int32)
    assert np.array_equal(got, CO.conv_replay(inp["initial_state"], res["state_update"],
                                              clamped).astype(np.float32))


def test_replay_zero_capacity_copies():
    inp = make_conv_inputs([1, 1, 1], 64, 4, "f32", seed=310)
    src = dev(inp["initial_state"], torch)
    acc = torch.zeros(3, dtype=torch.int32, device="cuda")
    _case("conv replay capacity 0")
    got = _replay(src, None, acc, 0)
    assert np.array_equal(got, inp["initial_state"])
