"""Host-side checks of the pooled entry points of libgdn.so (include/gdn_pool.h):
slot descriptions that break the slot rules are rejected on the host with the
documented status before anything is enqueued.

As in test_abi_host.py, every call here fails a host check (the fake device
addresses are never dereferenced) or has no work, and the module runs only
where no GPU is visible.
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

FAKE = 1 << 40
R, Hk, Hv, D, P = 3, 1, 2, 16, 6


def _tensors(same_pool=True):
    t = gdn.GdnTensors()
    addr = FAKE
    sizes = {"q": R * Hk * D * 2, "k": R * Hk * D * 2, "v": R * Hv * D * 2, "a": R * Hv * 4,
             "b": R * Hv * 4, "A_log": Hv * 4, "dt_bias": Hv * 4, "cu_seqlens": (R + 1) * 4,
             "initial_state": P * Hv * D * D * 4, "final_state": P * Hv * D * D * 4,
             "output": R * Hv * D * 2}
    for name, size in sizes.items():
        setattr(t, name, addr)
        addr += (size + 4095) // 4096 * 4096 + 4096
    if same_pool:
        t.final_state = t.initial_state
    return t, addr


def _slots(num=P, rd=None, wr=None, rd_host=None, wr_host=None):
    keep = []

    def host(x):
        if x is None:
            return None
        a = np.ascontiguousarray(np.asarray(x, np.int32))
        keep.append(a)
        return a.ctypes.data
    sl = gdn.GdnSlots(num, rd, wr, host(rd_host), host(wr_host))
    return sl, keep


def _forward(sl, t=None):
    t = t or _tensors()[0]
    p = gdn.make_params(R, R, Hk, Hv, D, D, gdn.GDN_F16, plan=gdn.PLAN_RECURRENT)
    return gdn.lib().gdn_forward_pooled(ctypes.byref(p), ctypes.byref(t),
                                        ctypes.byref(sl) if sl is not None else None, None, 0, None)


RD, WR = FAKE + (1 << 34), FAKE + (1 << 34) + 4096    # device slot arrays (never read)


def test_null_slots():
    assert _forward(None) == gdn.GDN_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(num=0), gdn.GDN_ERR_SHAPE),
    (dict(num=2), gdn.GDN_ERR_SHAPE),                                  # identity slots need R <= P
    (dict(rd=None, rd_host=[0, 1, 2], wr=WR), gdn.GDN_ERR_SHAPE),     # mirror of no array
    (dict(rd=RD, rd_host=[0, 1, P], wr=WR, wr_host=[3, 4, 5]), gdn.GDN_ERR_SHAPE),
    (dict(rd=RD, rd_host=[0, -2, 1], wr=WR, wr_host=[3, 4, 5]), gdn.GDN_ERR_SHAPE),
    (dict(rd=RD, rd_host=[0, 1, 2], wr=WR, wr_host=[3, 3, 5]), gdn.GDN_ERR_ALIAS),  # double write
    (dict(rd=RD, rd_host=[0, 1, 2], wr=WR, wr_host=[3, 0, 5]), gdn.GDN_ERR_ALIAS),  # writes another's read slot
    (dict(rd=None, wr=WR, wr_host=[1, 0, 2]), gdn.GDN_ERR_ALIAS),     # identity reads, crossed writes
])
def test_forward_slot_rules(kw, code):
    sl, keep = _slots(**kw)
    assert _forward(sl) == code


def test_forward_slot_arrays_must_not_overlap_outputs():
    t, _ = _tensors()
    sl, keep = _slots(rd=t.output, wr=WR)
    assert _forward(sl, t) == gdn.GDN_ERR_ALIAS


def test_conv_pooled_rules():
    t = gdn.GdnConvTensors()
    addr = FAKE
    C, K = 64, 4
    for name, size in {"x": R * C * 2, "weight": C * K * 4, "bias": C * 4, "cu_seqlens": (R + 1) * 4,
                       "initial_state": P * C * (K - 1) * 4, "output": R * C * 2}.items():
        setattr(t, name, addr)
        addr += (size + 4095) // 4096 * 4096 + 4096
    t.final_state = t.initial_state
    p = gdn.GdnConvParams(R, R, C, K, gdn.GDN_F16, gdn.CONV_SILU, 0)
    for kw, code in [(dict(wr=WR, wr_host=[2, 2, 4]), gdn.GDN_ERR_ALIAS),
                     (dict(num=0), gdn.GDN_ERR_SHAPE),
                     (dict(rd=RD, rd_host=[0, 1, 7], wr=WR, wr_host=[3, 4, 5]), gdn.GDN_ERR_SHAPE)]:
        sl, keep = _slots(**kw)
        assert gdn.lib().gdn_conv_forward_pooled(ctypes.byref(p), ctypes.byref(t), ctypes.byref(sl), None) == code
    assert gdn.lib().gdn_conv_forward_pooled(ctypes.byref(p), ctypes.byref(t), None, None) == gdn.GDN_ERR_NULL


def _replay(sl, src=FAKE, dst=FAKE, layout=gdn.STATE_V_MAJOR, params=True):
    cap = 2
    capsule = FAKE + (1 << 36)
    acc = FAKE + (1 << 37)
    p = gdn.make_params(0, R, Hk, Hv, D, D, gdn.GDN_F32, capacity=cap, state_layout=layout)
    return gdn.lib().gdn_replay_pooled(ctypes.byref(p) if params else None, src, capsule, acc, None, dst,
                                       ctypes.byref(sl) if sl is not None else None, None)


def test_replay_pooled_rules():
    sl, keep = _slots()
    assert _replay(sl, params=False) == gdn.GDN_ERR_NULL
    assert _replay(sl, layout=2) == gdn.GDN_ERR_SHAPE
    # without slots the states are request-indexed: one buffer for both is an overlap
    assert _replay(None) == gdn.GDN_ERR_ALIAS
    sl, keep = _slots(rd=RD, rd_host=[0, 1, 2], wr=WR, wr_host=[1, 4, 5])
    assert _replay(sl) == gdn.GDN_ERR_ALIAS                           # writes slot 1, read by request 1
    sl, keep = _slots(rd=RD, rd_host=[0, 1, 2], wr=WR, wr_host=[4, 4, 5])
    assert _replay(sl) == gdn.GDN_ERR_ALIAS
    sl, keep = _slots(rd=RD, wr=WR, wr_host=[3, 4, 9])
    assert _replay(sl) == gdn.GDN_ERR_SHAPE
    # one pool partly overlapping another is not one pool
    sl, keep = _slots(rd=RD, wr=WR)
    assert _replay(sl, src=FAKE, dst=FAKE + 256) == gdn.GDN_ERR_ALIAS


def test_conv_replay_pooled_rules():
    sl, keep = _slots(rd=RD, rd_host=[0, 1, 2], wr=WR, wr_host=[2, 4, 5])
    assert gdn.lib().gdn_conv_replay_pooled(R, 64, 4, 2, FAKE, FAKE + (1 << 36), FAKE + (1 << 37), None,
                                            FAKE, ctypes.byref(sl), None) == gdn.GDN_ERR_ALIAS


def test_publish_rules():
    L = gdn.lib()
    assert L.gdn_publish_slots(-1, FAKE, FAKE + 4096, None) == gdn.GDN_ERR_SHAPE
    assert L.gdn_publish_slots(0, None, None, None) == gdn.GDN_OK
    assert L.gdn_publish_slots(4, None, FAKE, None) == gdn.GDN_ERR_NULL
    assert L.gdn_publish_slots(4, FAKE, FAKE + 8, None) == gdn.GDN_ERR_ALIAS
