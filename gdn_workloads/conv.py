"""Seeded synthetic inputs for the compact causal convolution.

Like the rest of this package it only draws random numbers and casts them; it
holds none of the convolution's arithmetic. Shapes follow the compact
VarlenCausalConvWithState contract ("[CUDA] Add compact GatedDeltaNet
operator", the embedded VarlenCausalConv commit, Description): packed
token-major inputs, a [channels, kernel_size - 1] state per request and a
[batch, capacity, channels] capture.

  x             [N, C]          io dtype (float16 or float32), standard normal
  weight        [C, K]          float32, U(-1/sqrt(K), 1/sqrt(K)) (conv1d's default scale)
  bias          [C]             float32, same range
  initial_state [R, C, K - 1]   float32 standard normal (earlier inputs), or None
  capture_count [R]             int32 U{0 .. capacity + 1} (only when asked for;
                                capacity + 1 exercises the clamp)
  accepted      [R]             int32 U{0 .. capacity} (only when asked for)

Draw order (fixed, so a seed names the inputs exactly): lengths (when drawn),
x, weight, bias, initial state, capture counts, accepted.

The channel count of a hybrid layer's convolution is the width of the
concatenated q, k, v projections, 2 Hk Dk + Hv Dv: 8192 for Hk = 16, Hv = 32,
D = 128 and 10240 for Hv = 48.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import cu_from_lengths

__all__ = ["conv_channels", "make_conv_inputs"]


def conv_channels(Hk: int, Hv: int, Dk: int, Dv: int) -> int:
    return 2 * Hk * Dk + Hv * Dv


def make_conv_inputs(lengths: Optional[Sequence[int]], C: int, K: int, io_dtype: str, seed: int,
                     *, initial: str = "normal", capacity: int = 0, draw_counts: bool = False,
                     draw_accepted: bool = False, num_drawn: int = 0, max_drawn: int = 0) -> dict:
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(1, max_drawn + 1, num_drawn)
    lengths = np.asarray(lengths, dtype=np.int64)
    R = int(lengths.shape[0])
    N = int(lengths.sum())
    io = {"f32": np.float32, "f16": np.float16}[io_dtype]
    x = rng.standard_normal((N, C), dtype=np.float32).astype(io)
    bound = 1.0 / np.sqrt(K)
    weight = rng.uniform(-bound, bound, (C, K)).astype(np.float32)
    bias = rng.uniform(-bound, bound, C).astype(np.float32)
    if initial == "normal":
        initial_state = rng.standard_normal((R, C, K - 1), dtype=np.float32)
    elif initial == "zero":
        initial_state = None
    else:
        raise ValueError(f"unknown initial-state kind {initial!r}")
    capture_count = rng.integers(0, capacity + 2, R).astype(np.int32) if draw_counts else None
    accepted = rng.integers(0, capacity + 1, R).astype(np.int32) if draw_accepted else None
    return {"lengths": lengths, "cu_seqlens": cu_from_lengths(lengths), "x": x,
            "weight": weight, "bias": bias, "initial_state": initial_state,
            "capture_count": capture_count, "accepted": accepted, "C": C, "K": K,
            "io_dtype": io_dtype, "capacity": capacity}
