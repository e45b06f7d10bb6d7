"""Seeded synthetic inputs for the exact attention backward.

This module is shared by the oracle-side tests and by the GPU path's tests and
benchmark.  It holds no part of the attention arithmetic: it only draws random
tensors and builds the additive f16 masks (0 / -inf bit patterns), so that both
sides see exactly the same bytes.

Tensor layouts are ggml ``ne`` order (ne0 fastest), as in the ggmlR test file
"tests/testthat/test-flash-attn-back.R" (header comment of its ``attn_ref``):
    q [DK, N, H, B]   k [DK, M, Hkv, B]   v [DV, M, Hkv, B]   d [DV, H, N, B]
    mask [M, N] (f16, additive, shared by every head and batch)
A numpy array in ne order is stored here as a C-ordered array whose shape is the
ne shape reversed, e.g. q has numpy shape (B, H, N, DK).

Recipe (the pages print no seeds usable outside R): numpy.random.default_rng(seed),
draws taken in the order q, k, v, d, each a flat float64 array of prod(shape)
elements from uniform(-1, 1) (or standard normal where a workload asks for it),
cast to float32 and read in ne order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F16_NEG_INF = 0xFC00  # IEEE binary16 bit pattern of -inf
F16_ZERO = 0x0000


@dataclass(frozen=True)
class Shape:
    B: int
    H: int
    Hkv: int
    N: int
    M: int
    DK: int
    DV: int

    # numpy (C-order) shapes of the ne-order tensors
    @property
    def q_shape(self):
        return (self.B, self.H, self.N, self.DK)

    @property
    def k_shape(self):
        return (self.B, self.Hkv, self.M, self.DK)

    @property
    def v_shape(self):
        return (self.B, self.Hkv, self.M, self.DV)

    @property
    def d_shape(self):
        return (self.B, self.N, self.H, self.DV)

    @property
    def mask_shape(self):
        return (self.N, self.M)

    def astuple(self):
        return (self.B, self.H, self.Hkv, self.N, self.M, self.DK, self.DV)


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload."""
    name: str
    shape: Shape
    qk_dist: str  # "uniform" or "normal"
    vd_dist: str
    mask: str     # "none", "causal", "padding64"
    modes: tuple
    seed: int
    causal_metric: bool = False   # halve the counted FLOPs
    scale: float = field(default=0.0)

    def scale_f32(self) -> float:
        s = self.scale if self.scale else 1.0 / math.sqrt(self.shape.DK)
        return float(np.float32(s))


# The five workloads: shapes, distributions, masks and modes as specified for
# this path; seed = workload number.
WORKLOADS = {
    1: Workload("single-head B1 H1 N=M=128 D64 nomask", Shape(1, 1, 1, 128, 128, 64, 64),
                "uniform", "uniform", "none", ("f32",), 1),
    2: Workload("causal MHA B2 H8 N=M=1024 D64", Shape(2, 8, 8, 1024, 1024, 64, 64),
                "uniform", "uniform", "causal", ("f32", "bf16"), 2, True),
    3: Workload("causal GQA B1 H32/8 N=M=2048 D128", Shape(1, 32, 8, 2048, 2048, 128, 128),
                "uniform", "uniform", "causal", ("bf16",), 3, True),
    4: Workload("long-context causal GQA B1 H16/4 N=M=8192 D128", Shape(1, 16, 4, 8192, 8192, 128, 128),
                "normal", "uniform", "causal", ("bf16",), 4, True),
    5: Workload("padding-mask B4 H16 N512 M4096 DK192 DV128", Shape(4, 16, 16, 512, 4096, 192, 128),
                "uniform", "uniform", "padding64", ("f32", "bf16"), 5),
}


def _draw(rng: np.random.Generator, n: int, dist: str) -> np.ndarray:
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, n)
    elif dist == "normal":
        x = rng.standard_normal(n)
    else:
        raise ValueError(dist)
    return x.astype(np.float32)


def make_qkvd(shape: Shape, seed: int, qk_dist: str = "uniform", vd_dist: str = "uniform"):
    """Draw q, k, v, d (float32, numpy C-order shapes = reversed ne shapes)."""
    rng = np.random.default_rng(seed)
    s = shape
    q = _draw(rng, s.B * s.H * s.N * s.DK, qk_dist).reshape(s.q_shape)
    k = _draw(rng, s.B * s.Hkv * s.M * s.DK, qk_dist).reshape(s.k_shape)
    v = _draw(rng, s.B * s.Hkv * s.M * s.DV, vd_dist).reshape(s.v_shape)
    d = _draw(rng, s.B * s.H * s.N * s.DV, vd_dist).reshape(s.d_shape)
    return q, k, v, d


def causal_mask(N: int, M: int) -> np.ndarray:
    """f16 bits [M, N] in ne order (numpy shape (N, M)): 0 where key m <= query n, else -inf."""
    n = np.arange(N)[:, None]
    m = np.arange(M)[None, :]
    return np.where(m <= n, F16_ZERO, F16_NEG_INF).astype(np.uint16)


def padding64_mask(N: int, M: int, keep_keys: int = 3072, period: int = 64) -> np.ndarray:
    """Keys m >= keep_keys masked for every query; every key masked for queries n % period == 0."""
    n = np.arange(N)[:, None]
    m = np.arange(M)[None, :]
    masked = (m >= keep_keys) | (n % period == 0)
    return np.where(masked, F16_NEG_INF, F16_ZERO).astype(np.uint16)


def random_mask(N: int, M: int, seed: int, p_inf: float = 0.3, finite_scale: float = 2.0,
                full_rows: int = 1, full_cols: int = 1) -> np.ndarray:
    """A mask mixing finite additive values, -inf entries, all -inf rows and all -inf key columns."""
    rng = np.random.default_rng(seed + 7919)
    vals = rng.uniform(-finite_scale, finite_scale, (N, M)).astype(np.float16)
    bits = vals.view(np.uint16).copy()
    bits[rng.random((N, M)) < p_inf] = F16_NEG_INF
    if N > 0 and M > 0:
        for r in rng.choice(N, size=min(full_rows, N), replace=False):
            bits[r, :] = F16_NEG_INF
        for c in rng.choice(M, size=min(full_cols, M), replace=False):
            bits[:, c] = F16_NEG_INF
    return bits


def make_mask(kind: str, N: int, M: int, seed: int = 0):
    if kind == "none":
        return None
    if kind == "causal":
        return causal_mask(N, M)
    if kind == "padding64":
        return padding64_mask(N, M)
    if kind == "random":
        return random_mask(N, M, seed)
    raise ValueError(kind)


def workload_inputs(wid: int):
    """(shape, q, k, v, d, mask_bits_or_None, scale_f32) for one of the five workloads."""
    w = WORKLOADS[wid]
    q, k, v, d = make_qkvd(w.shape, w.seed, w.qk_dist, w.vd_dist)
    mask = make_mask(w.mask, w.shape.N, w.shape.M)
    return w.shape, q, k, v, d, mask, w.scale_f32()
