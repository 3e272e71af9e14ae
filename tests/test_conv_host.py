"""Host-side checks of the causal-convolution entry points of libgdn.so
(include/gdn_conv.h): every bad argument is rejected on the host with the
documented status before anything is enqueued.

As in test_abi_host.py, no call here launches a kernel: each one is built to
fail a host check (the fake device addresses are never dereferenced), or has no
work (R = 0), and the module runs only where no GPU is visible.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

import gateddeltanet_recurrence_amd as gdn


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0        # counts devices without initialising HIP
    except Exception:
        return False


pytestmark = [
    pytest.mark.skipif(not os.path.exists(gdn.library_path()),
                       reason="libgdn.so not built (run the build first)"),
    pytest.mark.skipif(_gpu_visible(), reason="fake-pointer host checks run only without a GPU"),
]

FAKE = 1 << 40          # 16-byte aligned, never dereferenced


def _tensors(N=16, R=2, C=64, K=4, io=2, cap=0, **override):
    sizes = {"x": N * C * io, "weight": C * K * 4, "bias": C * 4, "cu_seqlens": (R + 1) * 4,
             "initial_state": R * C * (K - 1) * 4, "final_state": R * C * (K - 1) * 4,
             "output": N * C * io}
    if cap:
        sizes["state_update"] = R * cap * C * 4
        sizes["capture_count"] = R * 4
    t = gdn.GdnConvTensors()
    addr = FAKE
    spans = {}
    for name, size in sizes.items():
        setattr(t, name, addr)
        spans[name] = (addr, size)
        addr += (size + 4095) // 4096 * 4096 + 4096
    for name, val in override.items():
        setattr(t, name, val)
    return t, spans


def _params(N=16, R=2, C=64, K=4, io=gdn.GDN_F16, act=gdn.CONV_SILU, cap=0):
    return gdn.GdnConvParams(N, R, C, K, io, act, cap)


def _forward(p, t):
    return gdn.lib().gdn_conv_forward(ctypes.byref(p) if p is not None else None,
                                      ctypes.byref(t) if t is not None else None, None)


def _bad_cu_host():
    """A host mirror that fails validation (cu[R] != N), so a call that would
    otherwise pass its checks still never reaches a launch."""
    return np.array([0, 3, 7], np.int32)


def test_null_structs():
    t, _ = _tensors()
    assert _forward(None, t) == gdn.GDN_ERR_NULL
    assert _forward(_params(), None) == gdn.GDN_ERR_NULL


@pytest.mark.parametrize("field,value,code", [
    ("activation", 2, gdn.GDN_ERR_RULE),
    ("activation", -1, gdn.GDN_ERR_RULE),
    ("io_dtype", gdn.GDN_BF16, gdn.GDN_ERR_DTYPE),
    ("channels", 6, gdn.GDN_ERR_SHAPE),            # not a multiple of 4
    ("channels", 0, gdn.GDN_ERR_SHAPE),
    ("kernel_size", 1, gdn.GDN_ERR_SHAPE),
    ("kernel_size", 9, gdn.GDN_ERR_SHAPE),
    ("num_tokens", -1, gdn.GDN_ERR_SHAPE),
    ("num_reqs", -1, gdn.GDN_ERR_SHAPE),
    ("state_update_capacity", -1, gdn.GDN_ERR_CAPACITY),
])
def test_param_validation(field, value, code):
    p = _params()
    setattr(p, field, value)
    t, _ = _tensors()
    assert _forward(p, t) == code


def test_empty_batch():
    t, _ = _tensors()
    assert _forward(_params(N=0, R=0), t) == gdn.GDN_OK      # nothing to do, nothing launched
    assert _forward(_params(N=4, R=0), t) == gdn.GDN_ERR_SHAPE


def test_capture_needs_capacity():
    t, _ = _tensors(cap=2)
    assert _forward(_params(cap=0), t) == gdn.GDN_ERR_CAPACITY


@pytest.mark.parametrize("name", ["x", "weight", "output"])
def test_required_pointers(name):
    t, _ = _tensors(**{name: None})
    assert _forward(_params(), t) == gdn.GDN_ERR_NULL


def test_dense_layout_rules():
    t, _ = _tensors(N=15, cu_seqlens=None)
    assert _forward(_params(N=15), t) == gdn.GDN_ERR_SHAPE          # 15 tokens over 2 requests
    host = np.array([0, 8, 16], np.int32)
    t, _ = _tensors(cu_seqlens=None, cu_seqlens_host=host.ctypes.data)
    assert _forward(_params(), t) == gdn.GDN_ERR_SHAPE              # a mirror of nothing


@pytest.mark.parametrize("name", ["x", "weight", "initial_state", "final_state", "output"])
def test_alignment(name):
    t, spans = _tensors()
    setattr(t, name, spans[name][0] + 8)
    assert _forward(_params(), t) == gdn.GDN_ERR_SHAPE


def test_capture_alignment():
    t, spans = _tensors(cap=2)
    t.state_update = spans["state_update"][0] + 4
    assert _forward(_params(cap=2), t) == gdn.GDN_ERR_SHAPE


@pytest.mark.parametrize("cu", [[1, 8, 16], [0, 9, 8], [0, 8, 15], [0, 8, 17]])
def test_malformed_host_cu(cu):
    host = np.array(cu, np.int32)
    t, _ = _tensors(cu_seqlens_host=host.ctypes.data)
    assert _forward(_params(), t) == gdn.GDN_ERR_SHAPE


@pytest.mark.parametrize("out_name,in_name", [
    ("output", "x"), ("output", "weight"), ("output", "initial_state"),
    ("final_state", "x"), ("final_state", "bias"), ("final_state", "cu_seqlens"),
    ("state_update", "x"), ("state_update", "initial_state"), ("state_update", "capture_count"),
    ("output", "final_state"), ("state_update", "output"),
])
def test_alias_rules(out_name, in_name):
    t, spans = _tensors(cap=2)
    setattr(t, out_name, spans[in_name][0])
    assert _forward(_params(cap=2), t) == gdn.GDN_ERR_ALIAS


def test_final_state_may_only_alias_initial_state_exactly():
    t, spans = _tensors()
    t.final_state = spans["initial_state"][0] + 16                   # partial overlap
    assert _forward(_params(), t) == gdn.GDN_ERR_ALIAS
    # the exact in-place form passes the alias rules; the bad mirror stops the call
    host = _bad_cu_host()
    t, spans = _tensors(cu_seqlens_host=host.ctypes.data)
    t.final_state = spans["initial_state"][0]
    assert _forward(_params(), t) == gdn.GDN_ERR_SHAPE


# ------------------------------------------------------------------ replay
def _replay(R=2, C=64, K=4, cap=3, src=FAKE, capture=FAKE + (1 << 24), accepted=FAKE + (2 << 24),
            accepted_host=None, dst=FAKE + (3 << 24)):
    return gdn.lib().gdn_conv_replay(R, C, K, cap, src, capture, accepted, accepted_host, dst, None)


@pytest.mark.parametrize("kw,code", [
    ({"R": -1}, gdn.GDN_ERR_SHAPE),
    ({"C": 10}, gdn.GDN_ERR_SHAPE),
    ({"K": 1}, gdn.GDN_ERR_SHAPE),
    ({"K": 9}, gdn.GDN_ERR_SHAPE),
    ({"cap": -1}, gdn.GDN_ERR_CAPACITY),
    ({"src": None}, gdn.GDN_ERR_NULL),
    ({"dst": None}, gdn.GDN_ERR_NULL),
    ({"accepted": None}, gdn.GDN_ERR_NULL),
    ({"capture": None}, gdn.GDN_ERR_NULL),
    ({"src": FAKE + 4}, gdn.GDN_ERR_SHAPE),
    ({"dst": FAKE + (3 << 24) + 8}, gdn.GDN_ERR_SHAPE),
    ({"capture": FAKE + (1 << 24) + 4}, gdn.GDN_ERR_SHAPE),
    ({"dst": FAKE + 64}, gdn.GDN_ERR_ALIAS),                      # inside src
    ({"dst": FAKE + (1 << 24)}, gdn.GDN_ERR_ALIAS),               # on the capture
    ({"dst": FAKE + (2 << 24)}, gdn.GDN_ERR_ALIAS),               # on accepted
])
def test_replay_validation(kw, code):
    assert _replay(**kw) == code


@pytest.mark.parametrize("acc", [[0, 4], [-1, 0]])
def test_replay_accepted_host_range(acc):
    host = np.array(acc, np.int32)
    assert _replay(accepted_host=host.ctypes.data) == gdn.GDN_ERR_CAPACITY


def test_replay_empty_batch():
    assert _replay(R=0, src=None, dst=None, accepted=None) == gdn.GDN_OK
