"""Seeded synthetic inputs and the workload table.

This module draws random numbers and rounds them to the input dtype; it holds none of retention's
arithmetic, so both the GPU library's callers and the fp64 oracle can take their inputs from it.

Inputs are generated as: numpy ``default_rng(seed)`` (PCG64) ``standard_normal`` in fp64, divided by the
workload's scale, cast to fp32, then rounded to bf16 (round to nearest, ties to even) when the workload is
bf16. The oracle consumes the already-rounded values, so a parity error measures the kernels only.

Per-head decay rates follow the multi-scale schedule gamma_h = 1 - 2^(-5-h) ("Hybrid Architectures: RetNet
and the Three Computation Paradigms", section 8.1; paper summary, multi-scale retention). The rotation
frequencies theta_i = 10000^(-2i/dk), i < dk/2, are the usual rotary choice; the pages only give the
theta = pi/4 illustration (blog section 6.9).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def gamma_schedule(h: int) -> np.ndarray:
    """gamma_h = 1 - 2^(-5-h) for h = 0..H-1, as fp32 (exact: 1 - 2^-k is representable for k <= 24)."""
    return (1.0 - np.exp2(-5.0 - np.arange(h, dtype=np.float64))).astype(np.float32)


def gamma_schedule_loglinear(h: int) -> np.ndarray:
    """The larger models' schedule gamma = 1 - exp(linspace(log 1/32, log 1/512, h)) ([Paper] summary, multi-scale
    retention): 1 - gamma runs geometrically from 1/32 to 1/512; fp32 (h >= 2)."""
    return (1.0 - np.exp(np.linspace(np.log(1.0 / 32), np.log(1.0 / 512), h))).astype(np.float32)


def theta_schedule(dk: int) -> np.ndarray:
    """theta_i = 10000^(-2i/dk) for i = 0..dk/2-1, fp64."""
    i = np.arange(dk // 2, dtype=np.float64)
    return np.power(10000.0, -2.0 * i / dk)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array rounded to the input dtype and returned as fp32 ('f32' leaves it unchanged)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x))
    raise ValueError(dtype)


def normal(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    return round_to((rng.standard_normal(shape) / scale).astype(np.float32), dtype)


@dataclass
class Workload:
    """One synthetic retention workload. Shapes follow [B, N, H, d] for q/k/v/o."""
    name: str
    B: int
    N: int
    H: int
    dk: int
    dv: int
    dtype: str              # input (and output) dtype: 'f32' or 'bf16'
    scale: float            # inputs ~ N(0,1)/scale
    seed: int
    chunk: int
    rotate: bool
    prefill: int = 0        # decode workloads: prefill length before the steps
    steps: int = 0          # decode workloads: number of single-token steps
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def gamma(self) -> np.ndarray:
        return gamma_schedule(self.H)

    @property
    def theta(self):
        return theta_schedule(self.dk) if self.rotate else None


# The five workloads this library is measured and checked on (sizes as stated for each).
WORKLOADS = {
    1: Workload("msr-fp32-tiny", B=1, N=64, H=8, dk=16, dv=16, dtype="f32", scale=1.0, seed=1, chunk=16,
                rotate=False, notes="parallel, recurrent and chunkwise (chunk 16) all checked"),
    2: Workload("retention-layer-d512", B=8, N=2048, H=8, dk=64, dv=64, dtype="bf16", scale=8.0, seed=2,
                chunk=64, rotate=True, notes="d_model=512 layer, chunkwise chunk 64"),
    3: Workload("batched-decode", B=128, N=512, H=8, dk=64, dv=64, dtype="bf16", scale=8.0, seed=3, chunk=64,
                rotate=True, prefill=512, steps=1024,
                notes="fp32 state from a 512-token chunkwise prefill, then 1024 single-token steps"),
    4: Workload("7b-class-layer", B=1, N=8192, H=16, dk=256, dv=512, dtype="bf16", scale=16.0, seed=4,
                chunk=128, rotate=True, notes="d_model=4096 layer, chunkwise chunk 128"),
    5: Workload("long-sequence", B=1, N=65536, H=8, dk=128, dv=128, dtype="bf16", scale=11.0, seed=5,
                chunk=128, rotate=True, prefill=65536, steps=256,
                notes="chunkwise chunk 128, final state handed to 256 decode steps"),
}


def make_qkv(w: Workload, rng: np.random.Generator | None = None):
    """Draw Q, K, V (in that order) for a whole sequence; values are fp32 holding the rounded inputs."""
    rng = rng if rng is not None else np.random.default_rng(w.seed)
    q = normal(rng, (w.B, w.N, w.H, w.dk), w.scale, w.dtype)
    k = normal(rng, (w.B, w.N, w.H, w.dk), w.scale, w.dtype)
    v = normal(rng, (w.B, w.N, w.H, w.dv), w.scale, w.dtype)
    return q, k, v, rng


def make_step(w: Workload, rng: np.random.Generator):
    """Draw one decode step's q, k ([B, H, dk]) and v ([B, H, dv]) in that order."""
    q = normal(rng, (w.B, w.H, w.dk), w.scale, w.dtype)
    k = normal(rng, (w.B, w.H, w.dk), w.scale, w.dtype)
    v = normal(rng, (w.B, w.H, w.dv), w.scale, w.dtype)
    return q, k, v


def make_dout(w: Workload, rng: np.random.Generator):
    """Draw an output gradient dL/dO ([B, N, H, dv]) for the gradient checks, drawn like V."""
    return normal(rng, (w.B, w.N, w.H, w.dv), w.scale, w.dtype)
