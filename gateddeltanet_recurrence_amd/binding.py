"""ctypes binding of the C ABI in include/gdn.h, include/gdn_conv.h and
include/gdn_pool.h (same entry-point names).

Tensors are torch tensors on the current HIP device; torch only provides the
device memory and the stream. Shapes are read from the tensors, checked for
consistency (the C ABI sees bare pointers and cannot), and passed as sizes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgdn.so"

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_ALIAS = 0, 1, 2, 3, 4
GDN_ERR_CAPACITY, GDN_ERR_WORKSPACE, GDN_ERR_PLAN, GDN_ERR_RULE, GDN_ERR_HIP = 5, 6, 7, 8, 9
GDN_ERR_SCRATCH = 10
NO_ALLOC_SCRATCH_BYTES = 128 << 20   # GDN_NO_ALLOC_SCRATCH_BYTES
GDN_F32, GDN_F16, GDN_BF16 = 0, 1, 2
PLAN_AUTO, PLAN_RECURRENT, PLAN_CHUNK = 0, 1, 2
RULE_GATED_DELTA, RULE_DELTA, RULE_GATED, RULE_LINEAR = 0, 1, 2, 3
GATE_RAW, GATE_NONE = 0, 1
STATE_V_MAJOR, STATE_K_MAJOR = 0, 1
ABI_VERSION = 7          # the struct layouts below match this version of include/gdn.h
CONV_SILU, CONV_NONE = 0, 1


class LibraryNotBuilt(RuntimeError):
    pass


class GDNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({gdn_strerror(status)})")


class GdnParams(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_reqs", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("chunk", ctypes.c_int32),
        ("state_update_capacity", ctypes.c_int32), ("plan", ctypes.c_int32),
        ("update_rule", ctypes.c_int32), ("gate_activation", ctypes.c_int32),
        ("state_layout", ctypes.c_int32),
    ]


class GdnTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "v", "a", "b", "A_log", "dt_bias", "cu_seqlens", "cu_seqlens_host",
        "initial_state", "final_state", "output", "state_update", "capture_count")]


class GdnConvParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "num_reqs", "channels", "kernel_size", "io_dtype", "activation",
        "state_update_capacity")]


class GdnConvTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "weight", "bias", "cu_seqlens", "cu_seqlens_host", "initial_state", "final_state",
        "output", "state_update", "capture_count")]


class GdnConvFused(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("mixed", "weight", "bias", "initial_state", "final_state")] + \
               [("kernel_size", ctypes.c_int32), ("activation", ctypes.c_int32)]


class GdnSlots(ctypes.Structure):
    _fields_ = [("num_slots", ctypes.c_int32), ("read_slots", ctypes.c_void_p),
                ("write_slots", ctypes.c_void_p), ("read_slots_host", ctypes.c_void_p),
                ("write_slots_host", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    """libgdn.so next to this file, or the file named by GDN_LIBRARY."""
    return os.environ.get("GDN_LIBRARY") or os.path.join(PKG, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so; raises LibraryNotBuilt when it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise LibraryNotBuilt(f"{path} is missing: build it with "
                                  "`python -m gateddeltanet_recurrence_amd.build`")
        L = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.gdn_forward.argtypes = [ctypes.POINTER(GdnParams), ctypes.POINTER(GdnTensors), vp,
                                  ctypes.c_size_t, vp]
        L.gdn_forward.restype = ctypes.c_int
        L.gdn_forward_no_alloc.argtypes = [ctypes.POINTER(GdnParams), ctypes.POINTER(GdnTensors), vp]
        L.gdn_forward_no_alloc.restype = ctypes.c_int
        L.gdn_forward_workspace_bytes.argtypes = [ctypes.POINTER(GdnParams), vp,
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_forward_workspace_bytes.restype = ctypes.c_int
        L.gdn_resolve_plan.argtypes = [ctypes.POINTER(GdnParams), vp, ctypes.POINTER(i32)]
        L.gdn_resolve_plan.restype = ctypes.c_int
        L.gdn_replay.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.gdn_replay.restype = ctypes.c_int
        L.gdn_replay_forward.argtypes = [ctypes.POINTER(GdnParams), ctypes.POINTER(GdnTensors), vp, vp, vp,
                                         vp, vp]
        L.gdn_replay_forward.restype = ctypes.c_int
        L.gdn_conv_forward.argtypes = [ctypes.POINTER(GdnConvParams),
                                       ctypes.POINTER(GdnConvTensors), vp]
        L.gdn_conv_forward.restype = ctypes.c_int
        L.gdn_conv_replay.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.gdn_conv_replay.restype = ctypes.c_int
        sp = ctypes.POINTER(GdnSlots)
        L.gdn_forward_pooled.argtypes = [ctypes.POINTER(GdnParams), ctypes.POINTER(GdnTensors), sp, vp,
                                         ctypes.c_size_t, vp]
        L.gdn_forward_pooled.restype = ctypes.c_int
        L.gdn_replay_pooled.argtypes = [ctypes.POINTER(GdnParams), vp, vp, vp, vp, vp, sp, vp]
        L.gdn_replay_pooled.restype = ctypes.c_int
        L.gdn_replay_forward_pooled.argtypes = [ctypes.POINTER(GdnParams), ctypes.POINTER(GdnTensors), sp, vp,
                                                vp, vp, vp, vp]
        L.gdn_replay_forward_pooled.restype = ctypes.c_int
        L.gdn_conv_forward_pooled.argtypes = [ctypes.POINTER(GdnConvParams),
                                              ctypes.POINTER(GdnConvTensors), sp, vp]
        L.gdn_conv_forward_pooled.restype = ctypes.c_int
        L.gdn_conv_replay_pooled.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, sp, vp]
        L.gdn_conv_replay_pooled.restype = ctypes.c_int
        L.gdn_conv_decode_forward.argtypes = [ctypes.POINTER(GdnParams), ctypes.POINTER(GdnTensors),
                                              ctypes.POINTER(GdnConvFused), vp]
        L.gdn_conv_decode_forward.restype = ctypes.c_int
        L.gdn_publish_slots.argtypes = [i32, vp, vp, vp]
        L.gdn_publish_slots.restype = ctypes.c_int
        L.gdn_strerror.argtypes = [ctypes.c_int]
        L.gdn_strerror.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = ctypes.c_int
        if L.gdn_abi_version() != ABI_VERSION:
            raise LibraryNotBuilt(f"{path} has ABI version {L.gdn_abi_version()}, this binding "
                                  f"needs {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def gdn_abi_version() -> int:
    return int(lib().gdn_abi_version())


def gdn_strerror(status: int) -> str:
    return lib().gdn_strerror(int(status)).decode()


def capsule_width(Hk: int, Hv: int, Dk: int, Dv: int) -> int:
    """Floats per capsule row: Hv decays, Hk*Dk unit keys, Hv*Dv deltas."""
    return Hv + Hk * Dk + Hv * Dv


def make_params(N, R, Hk, Hv, Dk, Dv, io_dtype, *, scale=0.0, chunk=0, capacity=0,
                plan=PLAN_AUTO, update_rule=RULE_GATED_DELTA, gate_activation=GATE_RAW,
                state_layout=STATE_V_MAJOR) -> GdnParams:
    return GdnParams(int(N), int(R), int(Hk), int(Hv), int(Dk), int(Dv), int(io_dtype),
                     float(scale), int(chunk), int(capacity), int(plan), int(update_rule),
                     int(gate_activation), int(state_layout))


# ------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


def _io_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return GDN_F32
    if dtype == torch.float16:
        return GDN_F16
    if dtype == torch.bfloat16:
        return GDN_BF16                      # passed through so the library rejects it
    raise ValueError(f"unsupported io dtype {dtype}")


def _ptr(x) -> Optional[int]:
    return None if x is None else int(x.data_ptr())


def _need(x, name, shape, dtype=None):
    if x is None:
        return
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)} != expected {tuple(shape)}")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype} != expected {dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return int(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _host_i32(arr):
    """Keep-alive int32 host buffer and its address, from a sequence / numpy / CPU tensor."""
    import numpy as np
    if arr is None:
        return None, None
    if hasattr(arr, "numpy") and hasattr(arr, "is_cuda"):
        if arr.is_cuda:
            raise ValueError("host mirrors must be CPU data")
        arr = arr.numpy()
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
    return a, a.ctypes.data


def _slots(R, num_slots, read_slots, write_slots, read_slots_host, write_slots_host):
    """GdnSlots for R requests plus the host arrays it points to (kept alive by the caller)."""
    torch = _torch()
    _need(read_slots, "read_slots", (R,), torch.int32)
    _need(write_slots, "write_slots", (R,), torch.int32)
    rh, rh_ptr = _host_i32(read_slots_host)
    wh, wh_ptr = _host_i32(write_slots_host)
    for h, name in ((rh, "read_slots_host"), (wh, "write_slots_host")):
        if h is not None and h.shape != (R,):
            raise ValueError(f"{name} must have R entries")
    sl = GdnSlots(int(num_slots), _ptr(read_slots), _ptr(write_slots), rh_ptr, wh_ptr)
    return sl, (rh, wh)


# ------------------------------------------------------------- entry points
def gdn_forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, **kw) -> int:
    """gdn_forward of include/gdn.h on torch tensors; returns the status code.
    Keywords as _forward."""
    return _forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, **kw)


def gdn_forward_no_alloc(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, **kw) -> int:
    """gdn_forward_no_alloc of include/gdn.h: gdn_forward whose workspace is the
    library's static scratch array on the current GPU (no workspace argument).
    Keywords as _forward, without workspace."""
    if kw.get("workspace") is not None:
        raise ValueError("gdn_forward_no_alloc takes no workspace")
    return _forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, no_alloc=True, **kw)


def gdn_replay_forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, *, prev_state_update,
                       accepted, replay_state, accepted_host=None, **kw) -> int:
    """gdn_replay_forward of include/gdn.h: replay of the previous step's accepted
    capsule prefix onto initial_state (the committed bank) into replay_state (the
    inactive bank) and the verify of this step's tokens from that state, in one
    pass. prev_state_update [R, capacity, W] float32, accepted [R] int32 (GPU
    tensors), accepted_host a host int32 mirror or None, replay_state
    [R, Hv, Dv, Dk] float32; the other keywords as _forward."""
    return _forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output,
                    replay=dict(prev=prev_state_update, accepted=accepted, state=replay_state,
                                accepted_host=accepted_host), **kw)


def gdn_replay_forward_pooled(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, *, num_slots: int,
                              prev_state_update, accepted, replay_pool, read_slots=None, write_slots=None,
                              read_slots_host=None, write_slots_host=None, accepted_host=None, **kw) -> int:
    """gdn_replay_forward_pooled of include/gdn_pool.h: initial_state and replay_pool
    are pools [P, Hv, Dv, Dk] (may be one tensor); request r replays from slot
    read_slots[r] into slot write_slots[r] and verifies from it."""
    pool = dict(num_slots=num_slots, read_slots=read_slots, write_slots=write_slots,
                read_slots_host=read_slots_host, write_slots_host=write_slots_host)
    return _forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, pool=pool,
                    replay=dict(prev=prev_state_update, accepted=accepted, state=replay_pool,
                                accepted_host=accepted_host), **kw)


def gdn_forward_pooled(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, *, num_slots: int,
                       read_slots=None, write_slots=None, read_slots_host=None,
                       write_slots_host=None, **kw) -> int:
    """gdn_forward_pooled of include/gdn_pool.h: initial_state and final_state are
    pools [P, Hv, Dv, Dk]; request r reads slot read_slots[r] and writes slot
    write_slots[r] (int32 GPU tensors [R], None for slot r)."""
    pool = dict(num_slots=num_slots, read_slots=read_slots, write_slots=write_slots,
                read_slots_host=read_slots_host, write_slots_host=write_slots_host)
    return _forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, pool=pool, **kw)


def _forward(q, k, v, a, b, A_log, dt_bias, cu_seqlens, output, *, initial_state=None,
             final_state=None, state_update=None, capture_count=None, cu_seqlens_host=None,
             scale: float = 0.0, chunk: int = 0, state_update_capacity: int = 0,
             plan: int = PLAN_AUTO, update_rule: int = RULE_GATED_DELTA,
             gate_activation: int = GATE_RAW, num_reqs: Optional[int] = None, workspace=None,
             stream=None, check: bool = True, pool=None, state_layout: int = STATE_V_MAJOR,
             no_alloc: bool = False, replay=None) -> int:
    """One forward call on torch tensors; returns the status code.

    q, k [N, Hk, Dk], v and output [N, Hv, Dv] in float16 or float32 (for the
    dense rank-4 layout, cu_seqlens None: [R, S, H, D] tensors, or the same
    flattened; R from num_reqs or the leading dim); a, b [N, Hv] float32 (raw
    gate inputs, or alpha and beta with gate_activation GATE_NONE, when A_log
    and dt_bias may be None); A_log, dt_bias [Hv] float32; cu_seqlens [R+1]
    int32 or None; states [R, Hv, Dv, Dk] float32; state_update
    [R, capacity, W] float32; capture_count [R] int32; workspace a uint8 GPU
    tensor (CHUNK plan).
    """
    torch = _torch()
    if cu_seqlens is None and q.dim() == 4:
        if num_reqs is None:
            num_reqs = q.shape[0]
        q, k, v, output = (x.reshape(-1, x.shape[2], x.shape[3]) for x in (q, k, v, output))
        a, b = (x.reshape(-1, x.shape[-1]) for x in (a, b))
    N, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    if cu_seqlens is None:
        if num_reqs is None:
            raise ValueError("the dense layout (cu_seqlens None) needs num_reqs or [R, S, H, D] inputs")
        R = int(num_reqs)
    else:
        R = cu_seqlens.shape[0] - 1
    io = q.dtype
    _need(q, "q", (N, Hk, Dk))
    _need(k, "k", (N, Hk, Dk), io)
    _need(v, "v", (N, Hv, Dv), io)
    _need(output, "output", (N, Hv, Dv), io)
    _need(a, "a", (N, Hv), torch.float32)
    _need(b, "b", (N, Hv), torch.float32)
    _need(A_log, "A_log", (Hv,), torch.float32)
    _need(dt_bias, "dt_bias", (Hv,), torch.float32)
    _need(cu_seqlens, "cu_seqlens", (R + 1,), torch.int32)
    S = int(pool["num_slots"]) if pool is not None else R
    st_shape = (S, Hv, Dk, Dv) if state_layout == STATE_K_MAJOR else (S, Hv, Dv, Dk)
    _need(initial_state, "initial_state", st_shape, torch.float32)
    _need(final_state, "final_state", st_shape, torch.float32)
    if state_update is not None:
        _need(state_update, "state_update",
              (R, state_update_capacity, capsule_width(Hk, Hv, Dk, Dv)), torch.float32)
    _need(capture_count, "capture_count", (R,), torch.int32)
    host_cu, host_cu_ptr = _host_i32(cu_seqlens_host)
    if host_cu is not None and host_cu.shape != (R + 1,):
        raise ValueError("cu_seqlens_host must have R + 1 entries")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        ws_ptr, ws_bytes = int(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    params = make_params(N, R, Hk, Hv, Dk, Dv, _io_code(io), scale=scale, chunk=chunk,
                         capacity=state_update_capacity, plan=plan, update_rule=update_rule,
                         gate_activation=gate_activation,
                         state_layout=state_layout)
    tens = GdnTensors(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                      _ptr(cu_seqlens), host_cu_ptr, _ptr(initial_state), _ptr(final_state),
                      _ptr(output), _ptr(state_update), _ptr(capture_count))
    where = "gdn_forward_pooled" if pool is not None else "gdn_forward"
    if replay is not None:
        if no_alloc or workspace is not None:
            raise ValueError("gdn_replay_forward takes no workspace")
        where = "gdn_replay_forward" if pool is None else "gdn_replay_forward_pooled"
        _need(replay["prev"], "prev_state_update",
              (R, state_update_capacity, capsule_width(Hk, Hv, Dk, Dv)), torch.float32)
        _need(replay["accepted"], "accepted", (R,), torch.int32)
        _need(replay["state"], "replay_state", st_shape, torch.float32)
        acc_host, acc_host_ptr = _host_i32(replay["accepted_host"])
        if acc_host is not None and acc_host.shape != (R,):
            raise ValueError("accepted_host must have R entries")
        if pool is None:
            st = lib().gdn_replay_forward(ctypes.byref(params), ctypes.byref(tens), _ptr(replay["prev"]),
                                          _ptr(replay["accepted"]), acc_host_ptr, _ptr(replay["state"]),
                                          _stream_handle(stream))
        else:
            sl, keep = _slots(R, **pool)
            st = lib().gdn_replay_forward_pooled(ctypes.byref(params), ctypes.byref(tens), ctypes.byref(sl),
                                                 _ptr(replay["prev"]), _ptr(replay["accepted"]), acc_host_ptr,
                                                 _ptr(replay["state"]), _stream_handle(stream))
            del keep
        del acc_host
    elif no_alloc:
        where = "gdn_forward_no_alloc"
        st = lib().gdn_forward_no_alloc(ctypes.byref(params), ctypes.byref(tens), _stream_handle(stream))
    elif pool is None:
        st = lib().gdn_forward(ctypes.byref(params), ctypes.byref(tens), ws_ptr,
                               ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    else:
        sl, keep = _slots(R, **pool)
        st = lib().gdn_forward_pooled(ctypes.byref(params), ctypes.byref(tens), ctypes.byref(sl), ws_ptr,
                                      ctypes.c_size_t(ws_bytes), _stream_handle(stream))
        del keep
    del host_cu
    if check and st != GDN_OK:
        raise GDNError(st, where)
    return st


def gdn_forward_workspace_bytes(N, R, Hk, Hv, Dk, Dv, io_dtype=GDN_F16, *, capacity=0,
                                plan=PLAN_AUTO, cu_seqlens_host=None, chunk=0) -> int:
    """Workspace bytes gdn_forward needs (0 for the recurrent plan)."""
    params = make_params(N, R, Hk, Hv, Dk, Dv, io_dtype, chunk=chunk, capacity=capacity, plan=plan)
    host_cu, host_ptr = _host_i32(cu_seqlens_host)
    out = ctypes.c_size_t(0)
    st = lib().gdn_forward_workspace_bytes(ctypes.byref(params), host_ptr, ctypes.byref(out))
    del host_cu
    if st != GDN_OK:
        raise GDNError(st, "gdn_forward_workspace_bytes")
    return int(out.value)


def gdn_resolve_plan(N, R, Hk, Hv, Dk, Dv, io_dtype=GDN_F16, *, capacity=0, plan=PLAN_AUTO,
                     cu_seqlens_host=None) -> int:
    params = make_params(N, R, Hk, Hv, Dk, Dv, io_dtype, capacity=capacity, plan=plan)
    host_cu, host_ptr = _host_i32(cu_seqlens_host)
    out = ctypes.c_int32(0)
    st = lib().gdn_resolve_plan(ctypes.byref(params), host_ptr, ctypes.byref(out))
    del host_cu
    if st != GDN_OK:
        raise GDNError(st, "gdn_resolve_plan")
    return int(out.value)


def gdn_replay(src_state, state_update, accepted, dst_state, *, num_k_heads: int,
               state_update_capacity: int, accepted_host=None, stream=None,
               check: bool = True) -> int:
    """gdn_replay of include/gdn.h: dst = src advanced by the accepted capsule prefix."""
    return _replay(src_state, state_update, accepted, dst_state, num_k_heads=num_k_heads,
                   state_update_capacity=state_update_capacity, accepted_host=accepted_host,
                   stream=stream, check=check)


def gdn_replay_pooled(src_pool, state_update, accepted, dst_pool, *, num_k_heads: int,
                      state_update_capacity: int, read_slots=None, write_slots=None,
                      read_slots_host=None, write_slots_host=None, accepted_host=None,
                      state_layout: int = STATE_V_MAJOR, pooled: bool = True, stream=None,
                      check: bool = True) -> int:
    """gdn_replay_pooled of include/gdn_pool.h: pools [P, Hv, Dv, Dk] (K-major
    [P, Hv, Dk, Dv]); the request count is accepted's length. pooled=False passes
    no slot description: the states are then [R, ...], indexed by request."""
    pool = None
    if pooled:
        pool = dict(num_slots=src_pool.shape[0], read_slots=read_slots, write_slots=write_slots,
                    read_slots_host=read_slots_host, write_slots_host=write_slots_host)
    return _replay(src_pool, state_update, accepted, dst_pool, num_k_heads=num_k_heads,
                   state_update_capacity=state_update_capacity, accepted_host=accepted_host,
                   stream=stream, check=check, pool=pool, state_layout=state_layout, via_params=True)


def _replay(src_state, state_update, accepted, dst_state, *, num_k_heads, state_update_capacity,
            accepted_host, stream, check, pool=None, state_layout=STATE_V_MAJOR, via_params=False):
    torch = _torch()
    if state_layout == STATE_K_MAJOR:
        S, Hv, Dk, Dv = src_state.shape
    else:
        S, Hv, Dv, Dk = src_state.shape
    R = accepted.shape[0]
    Hk = int(num_k_heads)
    cap = int(state_update_capacity)
    st_shape = tuple(src_state.shape)
    _need(dst_state, "dst_state", st_shape, torch.float32)
    _need(src_state, "src_state", st_shape, torch.float32)
    if pool is None and S != R:
        raise ValueError("request-indexed states need one state per request")
    _need(accepted, "accepted", (R,), torch.int32)
    if cap > 0:
        _need(state_update, "state_update", (R, cap, capsule_width(Hk, Hv, Dk, Dv)), torch.float32)
    host_acc, host_ptr = _host_i32(accepted_host)
    if host_acc is not None and host_acc.shape != (R,):
        raise ValueError("accepted_host must have R entries")
    if not via_params:
        st = lib().gdn_replay(R, Hk, Hv, Dk, Dv, cap, _ptr(src_state), _ptr(state_update),
                              _ptr(accepted), host_ptr, _ptr(dst_state), _stream_handle(stream))
    else:
        params = make_params(0, R, Hk, Hv, Dk, Dv, GDN_F32, capacity=cap, state_layout=state_layout)
        sl, keep = _slots(R, **pool) if pool is not None else (None, None)
        st = lib().gdn_replay_pooled(ctypes.byref(params), _ptr(src_state), _ptr(state_update),
                                     _ptr(accepted), host_ptr, _ptr(dst_state),
                                     ctypes.byref(sl) if sl is not None else None, _stream_handle(stream))
        del keep
    del host_acc
    if check and st != GDN_OK:
        raise GDNError(st, "gdn_replay_pooled" if via_params else "gdn_replay")
    return st


def gdn_conv_forward(x, weight, bias, cu_seqlens, output, **kw) -> int:
    """gdn_conv_forward of include/gdn_conv.h on torch tensors; returns the status.
    Keywords as _conv_forward."""
    return _conv_forward(x, weight, bias, cu_seqlens, output, **kw)


def gdn_conv_forward_pooled(x, weight, bias, cu_seqlens, output, *, num_slots: int, read_slots=None,
                            write_slots=None, read_slots_host=None, write_slots_host=None,
                            **kw) -> int:
    """gdn_conv_forward_pooled of include/gdn_pool.h: states are pools [P, C, K - 1]."""
    pool = dict(num_slots=num_slots, read_slots=read_slots, write_slots=write_slots,
                read_slots_host=read_slots_host, write_slots_host=write_slots_host)
    return _conv_forward(x, weight, bias, cu_seqlens, output, pool=pool, **kw)


def _conv_forward(x, weight, bias, cu_seqlens, output, *, initial_state=None,
                  final_state=None, state_update=None, capture_count=None,
                  cu_seqlens_host=None, activation: int = CONV_SILU,
                  state_update_capacity: int = 0, num_reqs: Optional[int] = None,
                  stream=None, check: bool = True, pool=None) -> int:
    """One convolution forward call on torch tensors; returns the status.

    x and output [N, C] float16 or float32 (dense layout, cu_seqlens None:
    [R, S, C] or [N, C] with num_reqs); weight [C, K] and bias [C] float32;
    cu_seqlens [R + 1] int32; states [R, C, K - 1] float32; state_update
    [R, capacity, C] float32; capture_count [R] int32.
    """
    torch = _torch()
    if cu_seqlens is None and x.dim() == 3:
        if num_reqs is None:
            num_reqs = x.shape[0]
        x, output = x.reshape(-1, x.shape[2]), output.reshape(-1, output.shape[2])
    N, C = x.shape
    K = weight.shape[1]
    if cu_seqlens is None:
        if num_reqs is None:
            raise ValueError("the dense layout (cu_seqlens None) needs num_reqs or [R, S, C] inputs")
        R = int(num_reqs)
    else:
        R = cu_seqlens.shape[0] - 1
    io = x.dtype
    _need(x, "x", (N, C))
    _need(output, "output", (N, C), io)
    _need(weight, "weight", (C, K), torch.float32)
    _need(bias, "bias", (C,), torch.float32)
    _need(cu_seqlens, "cu_seqlens", (R + 1,), torch.int32)
    S = int(pool["num_slots"]) if pool is not None else R
    _need(initial_state, "initial_state", (S, C, K - 1), torch.float32)
    _need(final_state, "final_state", (S, C, K - 1), torch.float32)
    if state_update is not None:
        _need(state_update, "state_update", (R, state_update_capacity, C), torch.float32)
    _need(capture_count, "capture_count", (R,), torch.int32)
    host_cu, host_cu_ptr = _host_i32(cu_seqlens_host)
    if host_cu is not None and host_cu.shape != (R + 1,):
        raise ValueError("cu_seqlens_host must have R + 1 entries")
    params = GdnConvParams(N, R, C, K, _io_code(io), int(activation), int(state_update_capacity))
    tens = GdnConvTensors(_ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens), host_cu_ptr,
                          _ptr(initial_state), _ptr(final_state), _ptr(output),
                          _ptr(state_update), _ptr(capture_count))
    if pool is None:
        st = lib().gdn_conv_forward(ctypes.byref(params), ctypes.byref(tens), _stream_handle(stream))
    else:
        sl, keep = _slots(R, **pool)
        st = lib().gdn_conv_forward_pooled(ctypes.byref(params), ctypes.byref(tens), ctypes.byref(sl),
                                           _stream_handle(stream))
        del keep
    del host_cu
    if check and st != GDN_OK:
        raise GDNError(st, "gdn_conv_forward_pooled" if pool is not None else "gdn_conv_forward")
    return st


def gdn_conv_decode_forward(mixed, conv_weight, conv_bias, a, b, A_log, dt_bias, cu_seqlens, output, *,
                            num_k_heads: int, head_k_dim: int, conv_initial_state=None, conv_final_state=None,
                            conv_activation: int = CONV_SILU, initial_state=None, final_state=None,
                            cu_seqlens_host=None, scale: float = 0.0, plan: int = PLAN_AUTO,
                            update_rule: int = RULE_GATED_DELTA, gate_activation: int = GATE_RAW,
                            num_reqs: Optional[int] = None, stream=None, check: bool = True) -> int:
    """gdn_conv_decode_forward of include/gdn_conv.h on torch tensors; returns the status.

    mixed [N, Cm] (dense layout, cu_seqlens None: [R, S, Cm]) float16 or float32,
    Cm = 2 Hk Dk + Hv Dv with the channels [q | k | v]; conv_weight [Cm, K] and
    conv_bias [Cm] float32; conv states [R, Cm, K - 1] float32; output [N, Hv, Dv]
    (or [R, S, Hv, Dv]) gives Hv and Dv; the rest as gdn_forward (V-major states).
    """
    torch = _torch()
    if cu_seqlens is None and mixed.dim() == 3:
        if num_reqs is None:
            num_reqs = mixed.shape[0]
        mixed = mixed.reshape(-1, mixed.shape[2])
        output = output.reshape(-1, output.shape[2], output.shape[3])
        a, b = (x.reshape(-1, x.shape[-1]) if x is not None else None for x in (a, b))
    N, Cm = mixed.shape
    Hv, Dv = output.shape[1], output.shape[2]
    Hk, Dk = int(num_k_heads), int(head_k_dim)
    if Cm != 2 * Hk * Dk + Hv * Dv:
        raise ValueError(f"mixed has {Cm} channels, expected 2 Hk Dk + Hv Dv = {2 * Hk * Dk + Hv * Dv}")
    K = conv_weight.shape[1]
    if cu_seqlens is None:
        if num_reqs is None:
            raise ValueError("the dense layout (cu_seqlens None) needs num_reqs or [R, S, Cm] inputs")
        R = int(num_reqs)
    else:
        R = cu_seqlens.shape[0] - 1
    io = mixed.dtype
    _need(mixed, "mixed", (N, Cm))
    _need(output, "output", (N, Hv, Dv), io)
    _need(conv_weight, "conv_weight", (Cm, K), torch.float32)
    _need(conv_bias, "conv_bias", (Cm,), torch.float32)
    _need(conv_initial_state, "conv_initial_state", (R, Cm, K - 1), torch.float32)
    _need(conv_final_state, "conv_final_state", (R, Cm, K - 1), torch.float32)
    _need(a, "a", (N, Hv), torch.float32)
    _need(b, "b", (N, Hv), torch.float32)
    _need(A_log, "A_log", (Hv,), torch.float32)
    _need(dt_bias, "dt_bias", (Hv,), torch.float32)
    _need(cu_seqlens, "cu_seqlens", (R + 1,), torch.int32)
    _need(initial_state, "initial_state", (R, Hv, Dv, Dk), torch.float32)
    _need(final_state, "final_state", (R, Hv, Dv, Dk), torch.float32)
    host_cu, host_cu_ptr = _host_i32(cu_seqlens_host)
    if host_cu is not None and host_cu.shape != (R + 1,):
        raise ValueError("cu_seqlens_host must have R + 1 entries")
    params = make_params(N, R, Hk, Hv, Dk, Dv, _io_code(io), scale=scale, plan=plan, update_rule=update_rule,
                         gate_activation=gate_activation)
    tens = GdnTensors(None, None, None, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens),
                      host_cu_ptr, _ptr(initial_state), _ptr(final_state), _ptr(output), None, None)
    conv = GdnConvFused(_ptr(mixed), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_initial_state),
                        _ptr(conv_final_state), int(K), int(conv_activation))
    st = lib().gdn_conv_decode_forward(ctypes.byref(params), ctypes.byref(tens), ctypes.byref(conv),
                                       _stream_handle(stream))
    del host_cu
    if check and st != GDN_OK:
        raise GDNError(st, "gdn_conv_decode_forward")
    return st


def gdn_conv_replay(src_state, state_update, accepted, dst_state, *, state_update_capacity: int,
                    accepted_host=None, stream=None, check: bool = True) -> int:
    """gdn_conv_replay of include/gdn_conv.h: dst = the last K - 1 of [src, accepted inputs]."""
    return _conv_replay(src_state, state_update, accepted, dst_state,
                        state_update_capacity=state_update_capacity, accepted_host=accepted_host,
                        stream=stream, check=check)


def gdn_conv_replay_pooled(src_pool, state_update, accepted, dst_pool, *, state_update_capacity: int,
                           read_slots=None, write_slots=None, read_slots_host=None,
                           write_slots_host=None, accepted_host=None, stream=None,
                           check: bool = True) -> int:
    """gdn_conv_replay_pooled of include/gdn_pool.h: pools [P, C, K - 1]."""
    pool = dict(num_slots=src_pool.shape[0], read_slots=read_slots, write_slots=write_slots,
                read_slots_host=read_slots_host, write_slots_host=write_slots_host)
    return _conv_replay(src_pool, state_update, accepted, dst_pool,
                        state_update_capacity=state_update_capacity, accepted_host=accepted_host,
                        stream=stream, check=check, pool=pool)


def _conv_replay(src_state, state_update, accepted, dst_state, *, state_update_capacity,
                 accepted_host, stream, check, pool=None):
    torch = _torch()
    S, C, Km1 = src_state.shape
    R = accepted.shape[0] if pool is not None else S
    cap = int(state_update_capacity)
    _need(src_state, "src_state", (S, C, Km1), torch.float32)
    _need(dst_state, "dst_state", (S, C, Km1), torch.float32)
    _need(accepted, "accepted", (R,), torch.int32)
    if cap > 0:
        _need(state_update, "state_update", (R, cap, C), torch.float32)
    host_acc, host_ptr = _host_i32(accepted_host)
    if host_acc is not None and host_acc.shape != (R,):
        raise ValueError("accepted_host must have R entries")
    if pool is None:
        st = lib().gdn_conv_replay(R, C, Km1 + 1, cap, _ptr(src_state), _ptr(state_update),
                                   _ptr(accepted), host_ptr, _ptr(dst_state), _stream_handle(stream))
    else:
        sl, keep = _slots(R, **pool)
        st = lib().gdn_conv_replay_pooled(R, C, Km1 + 1, cap, _ptr(src_state), _ptr(state_update),
                                          _ptr(accepted), host_ptr, _ptr(dst_state), ctypes.byref(sl),
                                          _stream_handle(stream))
        del keep
    del host_acc
    if check and st != GDN_OK:
        raise GDNError(st, "gdn_conv_replay_pooled" if pool is not None else "gdn_conv_replay")
    return st


def gdn_publish_slots(committed_slots, inactive_slots, *, stream=None, check: bool = True) -> int:
    """gdn_publish_slots of include/gdn_pool.h: exchanges the two int32 GPU slot arrays."""
    torch = _torch()
    R = committed_slots.shape[0]
    _need(committed_slots, "committed_slots", (R,), torch.int32)
    _need(inactive_slots, "inactive_slots", (R,), torch.int32)
    st = lib().gdn_publish_slots(R, _ptr(committed_slots), _ptr(inactive_slots), _stream_handle(stream))
    if check and st != GDN_OK:
        raise GDNError(st, "gdn_publish_slots")
    return st
