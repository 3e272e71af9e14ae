"""Host-side checks of libgdn.so: it loads, exports what include/*.h declare,
and rejects bad arguments on the host before anything reaches the GPU.

No call here launches a kernel: every forward/replay call is built to fail a
host-side check (fake device addresses are never dereferenced), and the
workspace / plan queries are host-only by contract.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import gateddeltanet_recurrence_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))



def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0        # counts devices without initialising HIP
    except Exception:
        return False


# Fake device addresses must never reach a real GPU: these host checks run only
# where no GPU is visible (a call that passed validation would launch a kernel).
pytestmark = [
    pytest.mark.skipif(not os.path.exists(gdn.library_path()),
                       reason="libgdn.so not built (run the build first)"),
    pytest.mark.skipif(_gpu_visible(), reason="fake-pointer host checks run only without a GPU"),
]


def declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_forward", "gdn_replay", "gdn_forward_workspace_bytes", "gdn_resolve_plan",
              "gdn_strerror", "gdn_abi_version", "gdn_conv_forward", "gdn_conv_replay"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_strerror():
    assert gdn.gdn_abi_version() == gdn.ABI_VERSION == 7
    assert gdn.gdn_strerror(gdn.GDN_OK) == "ok"
    assert "gdn_forward_no_alloc" in gdn.gdn_strerror(gdn.GDN_ERR_SCRATCH)
    assert "BF16" in gdn.gdn_strerror(gdn.GDN_ERR_DTYPE)
    assert gdn.gdn_strerror(12345) == "unknown status"


# -------------------------------------------------------- raw ABI helpers
FAKE = 1 << 40          # a 16-byte aligned address that is never dereferenced


def _tensors(N, R, Hk, Hv, Dk, Dv, io=2, **override):
    """Disjoint fake device ranges for every tensor of a forward call."""
    sizes = {"q": N * Hk * Dk * io, "k": N * Hk * Dk * io, "v": N * Hv * Dv * io,
             "a": N * Hv * 4, "b": N * Hv * 4, "A_log": Hv * 4, "dt_bias": Hv * 4,
             "cu_seqlens": (R + 1) * 4, "initial_state": R * Hv * Dv * Dk * 4,
             "final_state": R * Hv * Dv * Dk * 4, "output": N * Hv * Dv * io}
    t = gdn.GdnTensors()
    addr = FAKE
    for name, size in sizes.items():
        setattr(t, name, addr)
        addr += (size + 4095) // 4096 * 4096 + 4096
    for name, val in override.items():
        setattr(t, name, val)
    return t, addr


def _forward(params, tensors, ws=None, ws_bytes=0):
    return gdn.lib().gdn_forward(ctypes.byref(params), ctypes.byref(tensors), ws,
                                 ctypes.c_size_t(ws_bytes), None)


def _p(N=8, R=2, Hk=2, Hv=4, Dk=16, Dv=16, io=gdn.GDN_F16, **kw):
    return gdn.make_params(N, R, Hk, Hv, Dk, Dv, io, **kw)


def test_null_structs():
    t, _ = _tensors(8, 2, 2, 4, 16, 16)
    assert gdn.lib().gdn_forward(None, ctypes.byref(t), None, 0, None) == gdn.GDN_ERR_NULL
    p = _p()
    assert gdn.lib().gdn_forward(ctypes.byref(p), None, None, 0, None) == gdn.GDN_ERR_NULL


@pytest.mark.parametrize("field,value,code", [
    ("io_dtype", gdn.GDN_BF16, gdn.GDN_ERR_DTYPE),
    ("io_dtype", 7, gdn.GDN_ERR_DTYPE),
    ("update_rule", 4, gdn.GDN_ERR_RULE),
    ("update_rule", -1, gdn.GDN_ERR_RULE),
    ("gate_activation", 2, gdn.GDN_ERR_RULE),
    ("num_v_heads", 3, gdn.GDN_ERR_SHAPE),          # Hk = 2 does not divide 3
    ("head_k_dim", 48, gdn.GDN_ERR_SHAPE),
    ("head_v_dim", 256, gdn.GDN_ERR_SHAPE),
    ("num_tokens", -1, gdn.GDN_ERR_SHAPE),
    ("num_k_heads", 0, gdn.GDN_ERR_SHAPE),
    ("state_update_capacity", -1, gdn.GDN_ERR_CAPACITY),
    ("chunk", 32, gdn.GDN_ERR_SHAPE),
    ("plan", 9, gdn.GDN_ERR_PLAN),
    ("scale", float("nan"), gdn.GDN_ERR_SHAPE),
    ("state_layout", 2, gdn.GDN_ERR_SHAPE),
])
def test_param_validation(field, value, code):
    p = _p()
    setattr(p, field, value)
    t, _ = _tensors(8, 2, 2, 4, 16, 16)
    assert _forward(p, t) == code
    out = ctypes.c_size_t(0)
    assert gdn.lib().gdn_forward_workspace_bytes(ctypes.byref(p), None, ctypes.byref(out)) == code


def test_missing_required_pointers():
    for name in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "output"):
        t, _ = _tensors(8, 2, 2, 4, 16, 16, **{name: None})
        assert _forward(_p(), t) == gdn.GDN_ERR_NULL, name


def test_dense_layout_checks():
    # no cu_seqlens: every request holds N / R tokens
    t, _ = _tensors(7, 2, 2, 4, 16, 16, cu_seqlens=None)
    assert _forward(_p(N=7), t) == gdn.GDN_ERR_SHAPE             # 7 tokens do not split into 2
    t, _ = _tensors(8, 2, 2, 4, 16, 16, cu_seqlens=None)
    host = np.asarray([0, 4, 8], np.int32)
    t.cu_seqlens_host = host.ctypes.data
    assert _forward(_p(), t) == gdn.GDN_ERR_SHAPE                # a mirror of a missing array


def test_effective_gates_need_no_gate_parameters():
    # raw gates need A_log and dt_bias; effective gates (activation none) do not:
    # with them missing the call gets past the pointer checks to the next error
    t, _ = _tensors(8, 2, 2, 4, 16, 16, A_log=None, dt_bias=None)
    assert _forward(_p(), t) == gdn.GDN_ERR_NULL
    t.initial_state = t.initial_state + 4
    assert _forward(_p(gate_activation=gdn.GATE_NONE), t) == gdn.GDN_ERR_SHAPE


@pytest.mark.parametrize("rule,unread", [
    (gdn.RULE_DELTA, ("a", "A_log", "dt_bias")),           # ungated: no decay input
    (gdn.RULE_GATED, ("b",)),                              # no delta correction: no beta
    (gdn.RULE_LINEAR, ("a", "b", "A_log", "dt_bias")),
])
def test_rules_do_not_need_the_inputs_they_do_not_read(rule, unread):
    # with those inputs missing the call gets past the pointer checks to the next
    # error (a misaligned state); the gated delta rule needs them all
    t, _ = _tensors(8, 2, 2, 4, 16, 16, **{n: None for n in unread})
    t.initial_state = t.initial_state + 4
    assert _forward(_p(update_rule=rule), t) == gdn.GDN_ERR_SHAPE
    assert _forward(_p(update_rule=gdn.RULE_GATED_DELTA), t) == gdn.GDN_ERR_NULL


def test_rules_still_need_the_inputs_they_read():
    for rule, needed in ((gdn.RULE_DELTA, "b"), (gdn.RULE_GATED, "a"), (gdn.RULE_GATED, "A_log")):
        t, _ = _tensors(8, 2, 2, 4, 16, 16, **{needed: None})
        assert _forward(_p(update_rule=rule), t) == gdn.GDN_ERR_NULL, (rule, needed)


def test_tokens_without_requests_is_a_shape_error():
    t, _ = _tensors(8, 0, 2, 4, 16, 16)
    assert _forward(_p(N=8, R=0), t) == gdn.GDN_ERR_SHAPE
    assert _forward(_p(N=0, R=0), t) == gdn.GDN_OK           # nothing to do, nothing launched


def test_misaligned_state_is_rejected():
    t, _ = _tensors(8, 2, 2, 4, 16, 16)
    t.initial_state = t.initial_state + 4
    assert _forward(_p(), t) == gdn.GDN_ERR_SHAPE


@pytest.mark.parametrize("name", ["v", "output"])
def test_k_major_needs_aligned_v_and_output(name):
    # the K-major kernels move v and the output as 4-column vectors
    t, _ = _tensors(8, 2, 2, 4, 16, 16)
    setattr(t, name, getattr(t, name) + 2)
    assert _forward(_p(state_layout=gdn.STATE_K_MAJOR), t) == gdn.GDN_ERR_SHAPE


@pytest.mark.parametrize("cu,code", [
    ([1, 4, 8], gdn.GDN_ERR_SHAPE),      # must start at 0
    ([0, 5, 4], gdn.GDN_ERR_SHAPE),      # decreasing
    ([0, 4, 7], gdn.GDN_ERR_SHAPE),      # does not end at N = 8
])
def test_host_cu_seqlens_validation(cu, code):
    t, _ = _tensors(8, 2, 2, 4, 16, 16)
    host = np.asarray(cu, np.int32)
    t.cu_seqlens_host = host.ctypes.data
    assert _forward(_p(), t) == code


def test_alias_rules():
    N, R, Hk, Hv, Dk, Dv = 8, 2, 2, 4, 16, 16
    # output overlapping v
    t, _ = _tensors(N, R, Hk, Hv, Dk, Dv)
    t.output = t.v + 64
    assert _forward(_p(), t) == gdn.GDN_ERR_ALIAS
    # final_state partially overlapping initial_state
    t, _ = _tensors(N, R, Hk, Hv, Dk, Dv)
    t.final_state = t.initial_state + 1024
    assert _forward(_p(), t) == gdn.GDN_ERR_ALIAS
    # final_state over q
    t, _ = _tensors(N, R, Hk, Hv, Dk, Dv)
    t.final_state = t.q
    assert _forward(_p(), t) == gdn.GDN_ERR_ALIAS


def test_capsule_rules():
    N, R, Hk, Hv, Dk, Dv = 8, 2, 2, 4, 16, 16
    t, end = _tensors(N, R, Hk, Hv, Dk, Dv)
    t.state_update = end
    # a capsule with zero capacity has no rows to write
    assert _forward(_p(capacity=0), t) == gdn.GDN_ERR_CAPACITY
    # a capsule forces the recurrent path: a forced CHUNK plan is refused
    assert _forward(_p(Dk=128, Dv=128, capacity=4, plan=gdn.PLAN_CHUNK),
                    _tensors(N, R, Hk, Hv, 128, 128, state_update=end * 4)[0]) == gdn.GDN_ERR_PLAN
    # the capsule may not overlap the output
    t2, _ = _tensors(N, R, Hk, Hv, Dk, Dv)
    t2.state_update = t2.output
    assert _forward(_p(capacity=2), t2) == gdn.GDN_ERR_ALIAS


def test_plan_resolution_is_host_only():
    # capsule -> recurrent; small dims -> recurrent; forced recurrent honoured
    assert gdn.gdn_resolve_plan(64, 16, 16, 48, 128, 128, capacity=4) == gdn.PLAN_RECURRENT
    assert gdn.gdn_resolve_plan(4096, 1, 2, 2, 16, 16) == gdn.PLAN_RECURRENT
    assert gdn.gdn_resolve_plan(4096, 1, 16, 32, 128, 128, plan=gdn.PLAN_RECURRENT) == gdn.PLAN_RECURRENT
    assert gdn.gdn_resolve_plan(64, 64, 16, 32, 128, 128) == gdn.PLAN_RECURRENT
    assert gdn.gdn_forward_workspace_bytes(64, 64, 16, 32, 128, 128) == 0


def test_replay_validation():
    L = gdn.lib()
    src, cap, acc, dst = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    R, Hk, Hv, D = 2, 1, 2, 16
    assert L.gdn_replay(R, 2, 3, D, D, 4, src, cap, acc, None, dst, None) == gdn.GDN_ERR_SHAPE
    assert L.gdn_replay(R, Hk, Hv, 48, D, 4, src, cap, acc, None, dst, None) == gdn.GDN_ERR_SHAPE
    assert L.gdn_replay(R, Hk, Hv, D, D, -1, src, cap, acc, None, dst, None) == gdn.GDN_ERR_CAPACITY
    assert L.gdn_replay(R, Hk, Hv, D, D, 4, None, cap, acc, None, dst, None) == gdn.GDN_ERR_NULL
    assert L.gdn_replay(R, Hk, Hv, D, D, 4, src, None, acc, None, dst, None) == gdn.GDN_ERR_NULL
    assert L.gdn_replay(R, Hk, Hv, D, D, 4, src, cap, acc, None, src + 64, None) == gdn.GDN_ERR_ALIAS
    assert L.gdn_replay(R, Hk, Hv, D, D, 4, src, cap, acc, None, cap, None) == gdn.GDN_ERR_ALIAS
    bad = np.asarray([1, 5], np.int32)                       # 5 > capacity 4
    assert L.gdn_replay(R, Hk, Hv, D, D, 4, src, cap, acc, bad.ctypes.data, dst, None) == gdn.GDN_ERR_CAPACITY
    neg = np.asarray([-1, 0], np.int32)
    assert L.gdn_replay(R, Hk, Hv, D, D, 4, src, cap, acc, neg.ctypes.data, dst, None) == gdn.GDN_ERR_CAPACITY
    assert L.gdn_replay(0, Hk, Hv, D, D, 4, None, None, None, None, None, None) == gdn.GDN_OK


# ------------------------------------------- gdn_replay_forward (fused step)
def _fused_case(N=8, R=2, Hk=2, Hv=4, Dk=16, Dv=16, cap=4):
    """Fake disjoint ranges for a fused call: the forward tensors with a capsule,
    plus the previous capsule, accepted counts and the inactive bank."""
    t, addr = _tensors(N, R, Hk, Hv, Dk, Dv)
    W = Hv + Hk * Dk + Hv * Dv
    t.final_state = None
    t.state_update = addr
    addr += (R * cap * W * 4 + 4095) // 4096 * 4096 + 4096
    prev = addr
    addr += (R * cap * W * 4 + 4095) // 4096 * 4096 + 4096
    acc = addr
    addr += 4096
    dst = addr
    return t, prev, acc, dst, R * Hv * Dv * Dk * 4


def _fused(p, t, prev, acc, acc_host, dst):
    return gdn.lib().gdn_replay_forward(ctypes.byref(p), ctypes.byref(t), prev, acc, acc_host, dst, None)


def test_replay_forward_validation():
    t, prev, acc, dst, state_bytes = _fused_case()
    p = _p(capacity=4)
    # required pointers
    assert _fused(p, t, None, acc, None, dst) == gdn.GDN_ERR_NULL
    assert _fused(p, t, prev, None, None, dst) == gdn.GDN_ERR_NULL
    assert _fused(p, t, prev, acc, None, None) == gdn.GDN_ERR_NULL
    t2, *_ = _fused_case()
    t2.initial_state = None
    assert _fused(p, t2, prev, acc, None, dst) == gdn.GDN_ERR_NULL
    t3, *_ = _fused_case()
    t3.state_update = None
    assert _fused(p, t3, prev, acc, None, dst) == gdn.GDN_ERR_NULL
    # the K-major layout, a forced CHUNK plan, a misaligned inactive bank
    assert _fused(_p(capacity=4, state_layout=gdn.STATE_K_MAJOR), t, prev, acc, None, dst) \
        == gdn.GDN_ERR_SHAPE
    assert _fused(_p(capacity=4, plan=gdn.PLAN_CHUNK), t, prev, acc, None, dst) == gdn.GDN_ERR_PLAN
    assert _fused(p, t, prev, acc, None, dst + 4) == gdn.GDN_ERR_SHAPE
    # accepted_host beyond [0, capacity]
    for bad in ([5, 0], [-1, 2]):
        host = (ctypes.c_int32 * 2)(*bad)
        assert _fused(p, t, prev, acc, host, dst) == gdn.GDN_ERR_CAPACITY, bad
    # no request: nothing to do
    assert _fused(_p(N=0, R=0, capacity=4), t, prev, acc, None, dst) == gdn.GDN_OK


def test_replay_forward_aliasing():
    t, prev, acc, dst, state_bytes = _fused_case()
    p = _p(capacity=4)
    # the inactive bank may overlap nothing: the committed bank, the capsules,
    # the output, the counts
    for other in (t.initial_state, t.state_update, prev, t.output, acc, t.q):
        assert _fused(p, t, prev, acc, None, other) == gdn.GDN_ERR_ALIAS
    # the previous capsule is an input: it may not be the new one or the output
    assert _fused(p, t, t.state_update, acc, None, dst) == gdn.GDN_ERR_ALIAS
    assert _fused(p, t, t.output, acc, None, dst) == gdn.GDN_ERR_ALIAS
    # the committed bank is read only: no in-place final state
    t2, prev2, acc2, dst2, _ = _fused_case()
    t2.final_state = t2.initial_state
    assert _fused(p, t2, prev2, acc2, None, dst2) == gdn.GDN_ERR_ALIAS


def test_replay_forward_pooled_validation():
    t, prev, acc, dst, state_bytes = _fused_case()
    p = _p(capacity=4)
    L = gdn.lib()
    sl = gdn.GdnSlots()
    sl.num_slots = 4
    assert L.gdn_replay_forward_pooled(ctypes.byref(p), ctypes.byref(t), None, prev, acc, None, dst,
                                       None) == gdn.GDN_ERR_NULL
    # a final state is not taken with pools
    t2, prev2, acc2, dst2, _ = _fused_case()
    t2.final_state = dst2 + 8 * 4096 * 64
    assert L.gdn_replay_forward_pooled(ctypes.byref(p), ctypes.byref(t2), ctypes.byref(sl), prev2, acc2, None,
                                       dst2, None) == gdn.GDN_ERR_SHAPE
    # one pool: request 1 writes the slot request 0 reads (checked through the mirrors)
    rd = (ctypes.c_int32 * 2)(0, 1)
    wr = (ctypes.c_int32 * 2)(2, 0)
    sl.read_slots, sl.write_slots = FAKE - 8192, FAKE - 4096
    sl.read_slots_host = ctypes.cast(rd, ctypes.c_void_p)
    sl.write_slots_host = ctypes.cast(wr, ctypes.c_void_p)
    assert L.gdn_replay_forward_pooled(ctypes.byref(p), ctypes.byref(t), ctypes.byref(sl), prev, acc, None,
                                       t.initial_state, None) == gdn.GDN_ERR_ALIAS


def _conv_case(N=8, R=2, Hk=2, Hv=4, Dk=16, Dv=16, K=4, io=2):
    """Fake disjoint ranges for a fused convolution + decode call: the forward
    tensors without q, k, v, and the convolution's input, weights, bias and two
    state banks."""
    t, addr = _tensors(N, R, Hk, Hv, Dk, Dv)
    t.q = t.k = t.v = None
    Cm = 2 * Hk * Dk + Hv * Dv
    c = gdn.GdnConvFused()
    for name, size in (("mixed", N * Cm * io), ("weight", Cm * K * 4), ("bias", Cm * 4),
                       ("initial_state", R * Cm * (K - 1) * 4), ("final_state", R * Cm * (K - 1) * 4)):
        setattr(c, name, addr)
        addr += (size + 4095) // 4096 * 4096 + 4096
    c.kernel_size, c.activation = K, gdn.CONV_SILU
    return t, c


def _conv_decode(p, t, c):
    return gdn.lib().gdn_conv_decode_forward(ctypes.byref(p), ctypes.byref(t),
                                             ctypes.byref(c) if c is not None else None, None)


def test_conv_decode_validation():
    p = _p()
    t, c = _conv_case()
    assert _conv_decode(p, t, None) == gdn.GDN_ERR_NULL
    # q, k, v come from the convolution
    t2, c2 = _conv_case()
    t2.k = t.a
    assert _conv_decode(p, t2, c2) == gdn.GDN_ERR_SHAPE
    # kernel size 4 only; a known activation
    t2, c2 = _conv_case()
    c2.kernel_size = 3
    assert _conv_decode(p, t2, c2) == gdn.GDN_ERR_SHAPE
    c2.kernel_size, c2.activation = 4, 7
    assert _conv_decode(p, t2, c2) == gdn.GDN_ERR_RULE
    # no capsule, V-major only, never the CHUNK plan
    t2, c2 = _conv_case()
    t2.state_update = t2.output + (1 << 24)
    assert _conv_decode(_p(capacity=2), t2, c2) == gdn.GDN_ERR_SHAPE
    assert _conv_decode(_p(state_layout=gdn.STATE_K_MAJOR), t, c) == gdn.GDN_ERR_SHAPE
    assert _conv_decode(_p(Dk=128, Dv=128, plan=gdn.PLAN_CHUNK), *_conv_case(Dk=128, Dv=128)) \
        == gdn.GDN_ERR_PLAN
    # required convolution inputs when there are tokens
    for name in ("mixed", "weight"):
        t2, c2 = _conv_case()
        setattr(c2, name, None)
        assert _conv_decode(p, t2, c2) == gdn.GDN_ERR_NULL, name
    # 16-byte alignment of the vector-accessed convolution buffers
    for name in ("mixed", "weight", "initial_state", "final_state"):
        t2, c2 = _conv_case()
        setattr(c2, name, getattr(c2, name) + 4)
        assert _conv_decode(p, t2, c2) == gdn.GDN_ERR_SHAPE, name
    # no request: nothing to do
    assert _conv_decode(_p(N=0, R=0), t, c) == gdn.GDN_OK


def test_conv_decode_aliasing():
    p = _p()
    # the new carried inputs go to a bank of their own
    t, c = _conv_case()
    c.final_state = c.initial_state
    assert _conv_decode(p, t, c) == gdn.GDN_ERR_ALIAS
    for other in ("mixed", "weight", "bias"):
        t, c = _conv_case()
        c.final_state = getattr(c, other)
        assert _conv_decode(p, t, c) == gdn.GDN_ERR_ALIAS, other
    for other in ("output", "final_state", "initial_state", "a", "cu_seqlens"):
        t, c = _conv_case()
        c.final_state = getattr(t, other)
        assert _conv_decode(p, t, c) == gdn.GDN_ERR_ALIAS, other
    # outputs of the recurrence overlapping a convolution input
    for out in ("output", "final_state"):
        for inp in ("mixed", "weight", "initial_state"):
            t, c = _conv_case()
            setattr(t, out, getattr(c, inp))
            assert _conv_decode(p, t, c) == gdn.GDN_ERR_ALIAS, (out, inp)
