"""Seeded synthetic inputs for the selective-scan forward (generators only).

This module holds none of the method's arithmetic: it draws random tensors with
the shapes and value distributions of the workloads the pages discuss and
rounds them to the I/O precision.  Both the HIP path (via torch) and the CPU
oracle consume the same arrays.

Recipe (the same for every workload unless stated):
  * numpy ``default_rng(seed)`` (PCG64), fp32 draws, in the order
    x, z_delta, B, C, D_skip, then valid_len;
  * x ~ N(0, 1) [batch, L, dim];
  * delta_raw = 0.5 * z_delta + bias, z_delta ~ N(0, 1) [batch, L, dim]
    (the kernel applies softplus, so delta = softplus(N(0,1)*0.5 + bias));
  * A_log[d, n] = log(n + 1) [dim, dstate] (so A = -(n + 1));
  * B, C ~ N(0, 1) [batch, L, dstate], shared by all channels of a row;
  * D_skip ~ N(0, 1) [dim];
  * valid_len: all L, or uniform integers in [lo, L] (inclusive);
  * for bf16 I/O, x, delta_raw, B and C are rounded to bf16 (round to nearest
    even) and kept as float32 arrays holding exactly those bf16 values.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io: str                      # "f32" or "bf16"
    delta_bias: float = -4.0
    delta_clamp: tuple | None = None
    varlen_lo: int | None = None  # None: every row has seqlen valid steps

    def updates(self, valid_len=None) -> int:
        """State updates of one forward: sum over rows of valid steps * dim * dstate."""
        steps = self.batch * self.seqlen if valid_len is None else int(np.sum(valid_len))
        return steps * self.dim * self.dstate


WORKLOADS = {
    0: Workload("tiny-f32-b2-l256-d64-n16", 2, 256, 64, 16, "f32"),
    1: Workload("bf16-b8-l2048-d2048-n16", 8, 2048, 2048, 16, "bf16"),
    2: Workload("bf16-b8-l4096-d1024-n16", 8, 4096, 1024, 16, "bf16"),
    3: Workload("varlen-bf16-b16-l8192-d512-n16", 16, 8192, 512, 16, "bf16", varlen_lo=128),
    4: Workload("long-bf16-b1-l32768-d2048-n64", 1, 32768, 2048, 64, "bf16", delta_bias=-5.0,
                delta_clamp=(1e-3, 0.1)),
}

HEADLINE = 2


def seed_for(index: int) -> int:
    return 1000 + index


def round_to_bf16(a) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding the bf16 value.
    (For finite inputs the 32-bit sum below cannot wrap; NaNs become a quiet NaN.)"""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = u + np.uint32(0x7FFF)
    r += lsb
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC00000
    return r.view(np.float32).reshape(a.shape)


def bf16_bits(a) -> np.ndarray:
    """The 16-bit patterns of fp32 values that are exactly bf16."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def make_inputs(w: Workload, seed: int, with_D: bool = True) -> dict:
    """Draw one input set for workload ``w``.  Returns numpy arrays:
    x, delta, B, C (float32, bf16-exact when w.io == 'bf16'), A_log [dim, dstate]
    float32, D [dim] float32 or None, valid_len [batch] int32 or None."""
    rng = np.random.default_rng(seed)
    shp = (w.batch, w.seqlen, w.dim)
    x = rng.standard_normal(shp, dtype=np.float32)
    z = rng.standard_normal(shp, dtype=np.float32)
    delta = (z * np.float32(0.5) + np.float32(w.delta_bias)).astype(np.float32)
    del z
    B = rng.standard_normal((w.batch, w.seqlen, w.dstate), dtype=np.float32)
    C = rng.standard_normal((w.batch, w.seqlen, w.dstate), dtype=np.float32)
    D = rng.standard_normal((w.dim,), dtype=np.float32)
    valid_len = None
    if w.varlen_lo is not None:
        valid_len = rng.integers(w.varlen_lo, w.seqlen, endpoint=True, size=w.batch).astype(np.int32)
    A_log = np.broadcast_to(np.log(np.arange(1, w.dstate + 1, dtype=np.float64)).astype(np.float32),
                            (w.dim, w.dstate)).copy()
    if w.io == "bf16":
        x, delta, B, C = (round_to_bf16(v) for v in (x, delta, B, C))
    return dict(x=x, delta=delta, A_log=A_log, B=B, C=C, D=D if with_D else None, valid_len=valid_len)


def small_workload(base: Workload, batch=None, seqlen=None, dim=None) -> Workload:
    """The same recipe at another size (for parity cases the oracle finishes quickly)."""
    return dataclasses.replace(base, name=base.name + "-small", batch=batch or base.batch,
                               seqlen=seqlen or base.seqlen, dim=dim or base.dim)


def make_cotangents(w: Workload, seed: int) -> dict:
    """Seeded gradients of the outputs for the backward: dy [batch, L, dim]
    ~ N(0, 1) (bf16-exact for bf16 I/O) and dh_last [batch, dim, dstate]
    ~ N(0, 1) fp32, drawn in that order from their own generator."""
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((w.batch, w.seqlen, w.dim), dtype=np.float32)
    dh_last = rng.standard_normal((w.batch, w.dim, w.dstate), dtype=np.float32)
    if w.io == "bf16":
        dy = round_to_bf16(dy)
    return dict(dy=dy, dh_last=dh_last)
