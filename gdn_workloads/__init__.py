"""Seeded synthetic inputs for the GatedDeltaNet operator.

This module is shared by the float64 oracle's tests, the GPU parity tests and
the benchmark. It only draws random numbers and casts them to the dtypes the
operator takes; it holds none of the operator's arithmetic.

Shapes follow the operator contract described on "[CUDA] Add compact
GatedDeltaNet operator" (Description: packed ragged inputs, three outputs) and
"Add GatedDeltaNet evaluation export for Qwen hybrid models" (What changed:
packed THD q/k/v with cumulative sequence lengths, FP32 gate ABI, FP32 V-major
state):

  q, k          [N, Hk, Dk]       io dtype (float16 or float32)
  v             [N, Hv, Dv]       io dtype
  a, b          [N, Hv]           float32 raw gate inputs
  A_log, dt_bias [Hv]             float32, one scalar per value head
  cu_seqlens    [R + 1]           int32
  initial_state [R, Hv, Dv, Dk]   float32 (or None for a zero state)
  accepted      [R]               int32 accepted-prefix lengths (replay only)

Draw order for one workload (fixed, so a seed names the inputs exactly):
  1. sequence lengths (only when they are drawn)
  2. q, k, v    standard normal
  3. a, b       standard normal
  4. A_log = log(U[1, 16]) per value head
  5. dt_bias ~ U[-1, 1] per value head
  6. initial state ~ N(0, 0.05) (standard deviation 0.05), when nonzero
  7. accepted ~ U{0 .. capacity} per request (only when asked for)
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "workload_inputs", "cu_from_lengths"]


@dataclass(frozen=True)
class Workload:
    """One named synthetic workload of the operator."""

    name: str
    seed: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    io_dtype: str                     # "f32" or "f16"
    lengths: Optional[tuple] = None   # fixed per-request lengths, or None to draw
    num_drawn: int = 0                # number of lengths drawn from U[1, max_drawn]
    max_drawn: int = 0
    initial: str = "normal"           # "normal" (N(0, 0.05)) or "zero"
    capacity: int = 0                 # state_update capacity (0: no capsule)
    draw_accepted: bool = False
    description: str = ""

    def resolve_lengths(self, rng: np.random.Generator) -> np.ndarray:
        if self.lengths is not None:
            return np.asarray(self.lengths, dtype=np.int64)
        return rng.integers(1, self.max_drawn + 1, self.num_drawn).astype(np.int64)


WORKLOADS = {
    "tiny_recurrent": Workload(
        name="tiny_recurrent", seed=0, Hk=2, Hv=2, Dk=16, Dv=16, io_dtype="f32",
        lengths=(16,), initial="zero",
        description="1 sequence, T=16, Hk=Hv=2, Dk=Dv=16, fp32, zero initial state"),
    "batched_decode": Workload(
        name="batched_decode", seed=1, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype="f16",
        lengths=(1,) * 64,
        description="64 requests x T=1, Hk=16, Hv=32, D=128, fp16, state N(0,0.05), in place"),
    "ragged_prefill": Workload(
        name="ragged_prefill", seed=3, Hk=16, Hv=32, Dk=128, Dv=128, io_dtype="f16",
        num_drawn=8, max_drawn=4096,
        description="8 sequences, lengths U[1,4096] (seed 3), Hk=16, Hv=32, D=128, fp16"),
    "spec_verify_replay": Workload(
        name="spec_verify_replay", seed=4, Hk=16, Hv=48, Dk=128, Dv=128, io_dtype="f16",
        lengths=(4,) * 16, capacity=4, draw_accepted=True,
        description="16 requests x 4 draft tokens, Hk=16, Hv=48, D=128, fp16, capacity 4"),
    "long_prefill": Workload(
        name="long_prefill", seed=5, Hk=16, Hv=48, Dk=128, Dv=128, io_dtype="f16",
        lengths=(32768,),
        description="1 sequence, T=32768, Hk=16, Hv=48, D=128, fp16"),
}


def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """Cumulative sequence lengths [R + 1] (int32) of per-request lengths."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("packed token count does not fit int32")
    return cu.astype(np.int32)


def _np_io(io_dtype: str):
    if io_dtype == "f32":
        return np.float32
    if io_dtype == "f16":
        return np.float16
    raise ValueError(f"unsupported io dtype {io_dtype!r}")


def make_inputs(lengths: Optional[Sequence[int]], Hk: int, Hv: int, Dk: int, Dv: int,
                io_dtype: str, seed: int, *, initial: str = "normal",
                capacity: int = 0, draw_accepted: bool = False,
                num_drawn: int = 0, max_drawn: int = 0) -> dict:
    """Draw one set of operator inputs in the fixed order documented above.

    Returns a dict of numpy arrays in the dtypes the operator takes; "lengths"
    and "cu_seqlens" describe the packing. Large arrays are drawn in float32.
    """
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(1, max_drawn + 1, num_drawn)
    lengths = np.asarray(lengths, dtype=np.int64)
    R = int(lengths.shape[0])
    N = int(lengths.sum())
    io = _np_io(io_dtype)
    q = rng.standard_normal((N, Hk, Dk), dtype=np.float32).astype(io)
    k = rng.standard_normal((N, Hk, Dk), dtype=np.float32).astype(io)
    v = rng.standard_normal((N, Hv, Dv), dtype=np.float32).astype(io)
    a = rng.standard_normal((N, Hv), dtype=np.float32)
    b = rng.standard_normal((N, Hv), dtype=np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, Hv)).astype(np.float32)
    dt_bias = rng.uniform(-1.0, 1.0, Hv).astype(np.float32)
    if initial == "normal":
        initial_state = (rng.standard_normal((R, Hv, Dv, Dk), dtype=np.float32)
                         * np.float32(0.05))
    elif initial == "zero":
        initial_state = None
    else:
        raise ValueError(f"unknown initial-state kind {initial!r}")
    accepted = None
    if draw_accepted:
        accepted = rng.integers(0, capacity + 1, R).astype(np.int32)
    return {
        "lengths": lengths, "cu_seqlens": cu_from_lengths(lengths),
        "q": q, "k": k, "v": v, "a": a, "b": b, "A_log": A_log, "dt_bias": dt_bias,
        "initial_state": initial_state, "accepted": accepted,
        "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv, "io_dtype": io_dtype,
        "capacity": capacity,
    }


def workload_inputs(name: str) -> dict:
    """Inputs of one named workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    return make_inputs(w.lengths, w.Hk, w.Hv, w.Dk, w.Dv, w.io_dtype, w.seed,
                       initial=w.initial, capacity=w.capacity,
                       draw_accepted=w.draw_accepted, num_drawn=w.num_drawn,
                       max_drawn=w.max_drawn)
