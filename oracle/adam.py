"""Oracle (test infrastructure only): the host optimiser step and the low-precision refresh.

MegaTrain summary page, 方法步骤详情 phase 4: the optimiser update theta <- AdamUpdate(theta, grad,
m, v) runs on the CPU over the host-resident fp32 state. The RoundPipe popular article (§五) keeps
three copies of every parameter: a transient GPU compute copy, a low-precision host copy and a
high-precision optimiser copy; ``bf16_round`` is the refresh of the low-precision copy.

The pages do not state the Adam constants. Reading: beta1 = 0.9, beta2 = 0.999, eps = 1e-8, no
weight decay, step counter t starting at 1. The per-element arithmetic is written in float32 in
this exact order, with the bias corrections 1 - beta^t formed in fp64 and rounded to float32 once
per step, so that any implementation following the same order agrees bit for bit:

    m     = b1 * m + (1 - b1) * g
    v     = b2 * v + (1 - b2) * (g * g)
    mhat  = m / bc1                 bc1 = f32(1 - b1^t)
    vhat  = v / bc2                 bc2 = f32(1 - b2^t)
    theta = theta - (lr * mhat) / (sqrt(vhat) + eps)

where b1, b2, lr and eps are the configured values rounded to float32 (a configuration holds
them as float32), and (1 - b1), (1 - b2), bc1, bc2 are formed in fp64 from those float32 values
and rounded to float32 once.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def adam_constants(t: int, lr: float, b1: float, b2: float, eps: float):
    b1d, b2d = float(F32(b1)), float(F32(b2))
    return dict(b1=F32(b1), b2=F32(b2), omb1=F32(1.0 - b1d), omb2=F32(1.0 - b2d),
                bc1=F32(1.0 - b1d ** t), bc2=F32(1.0 - b2d ** t), lr=F32(lr), eps=F32(eps))


def adam_update(theta: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, t: int,
                lr: float = 1e-3, b1: float = 0.9, b2: float = 0.999, eps: float = 1e-8) -> None:
    """In-place float32 Adam step number ``t`` (t >= 1) on one tensor."""
    assert theta.dtype == g.dtype == m.dtype == v.dtype == np.float32
    c = adam_constants(t, lr, b1, b2, eps)
    m[...] = c["b1"] * m + c["omb1"] * g
    v[...] = c["b2"] * v + c["omb2"] * (g * g)
    mhat = m / c["bc1"]
    vhat = v / c["bc2"]
    theta[...] = theta - (c["lr"] * mhat) / (np.sqrt(vhat) + c["eps"])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16) by round-to-nearest-even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
