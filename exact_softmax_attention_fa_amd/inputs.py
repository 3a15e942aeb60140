"""Seeded synthetic inputs for the attention forward pass.

This module holds no attention arithmetic. It draws random numbers, rounds the
draws to the storage format of the workload (fp32, or bf16 by round-to-nearest-even),
and describes each workload's shape, scale and mask. Both the GPU path and the
CPU oracle consume exactly the arrays produced here, so the two always see the
same stored bits.

Workloads follow the shapes the pages use: N=4096 score tables and 64x64 tiles
(interactiveml.org, "FlashAttention saves the matrix, not the quadratic work"),
N=8192 with two-byte elements (lihaoran.work, "The intermediate matrix comes
first"), 32K contexts (sadullah.online, "Why this matters beyond raw speed"),
and scalar examples with one value column (lihaoran.work "Check three scores";
liminalml.com, executable scalar-value example).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    The draws here are finite normals, so NaN handling is not needed; an infinite or
    NaN input raises instead of being rounded silently.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding of non-finite input is not supported")
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    """Shape and storage description of one attention forward call."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16": storage of q, k, v and o
    causal: bool
    seed: int
    k_std: float = 1.0
    boost_frac: float = 0.0   # fraction of keys that get a common logit offset
    boost_logit: float = 0.0  # size of that offset, in scaled-score units
    note: str = ""
    scale: float = field(default=float("nan"))

    def resolved_scale(self) -> float:
        return 1.0 / math.sqrt(self.d) if math.isnan(self.scale) else self.scale

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d (two products of 2*N^2*d flops per head), halved for causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Read q, k, v once, write o once (input dtype) and lse once (fp32)."""
        n = self.B * self.H * self.N
        return 4 * n * self.d * self.elem_bytes + 4 * n


# The five workloads. Seeds are 1000 + workload index.
WORKLOADS = {
    "fwd_f32_b1_h1_n256_d64": Workload(
        "fwd_f32_b1_h1_n256_d64", 1, 1, 256, 64, "f32", False, 1001,
        note="single head, fp32 N(0,1) inputs, unmasked"),
    "fwd_bf16_b2_h8_n1024_d64": Workload(
        "fwd_bf16_b2_h8_n1024_d64", 2, 8, 1024, 64, "bf16", False, 1002,
        note="bf16 N(0,1) inputs, unmasked"),
    "fwd_bf16_b4_h16_n4096_d128_causal": Workload(
        "fwd_bf16_b4_h16_n4096_d128_causal", 4, 16, 4096, 128, "bf16", True, 1003,
        note="bf16 N(0,1) inputs, causal (key j <= query i)"),
    "fwd_bf16_b1_h16_n8192_d128_widek": Workload(
        "fwd_bf16_b1_h16_n8192_d128_widek", 1, 16, 8192, 128, "bf16", False, 1004,
        k_std=3.0, boost_frac=0.01, boost_logit=8.0,
        note="bf16, K ~ N(0,3^2), +8 logit offset on 1% of keys, unmasked"),
    "fwd_bf16_b1_h8_n32768_d128_causal": Workload(
        "fwd_bf16_b1_h8_n32768_d128_causal", 1, 8, 32768, 128, "bf16", True, 1005,
        note="bf16 N(0,1) inputs, causal, long context in one pass"),
}

# Workload whose throughput is the headline figure.
HEADLINE = "fwd_bf16_b1_h16_n8192_d128_widek"

# Measurement-only shapes (not parity configurations of their own; the GPU tests cover their
# kernels at smaller sizes): the head-width sweep at the headline's B, H, N with plain N(0,1)
# inputs, and single heads of long sequences, where one query-tile column leaves most of the
# chip idle and the key range is split over workgroups.
EXTRA_WORKLOADS = {
    **{f"sweep_bf16_b1_h16_n8192_d{d}": Workload(
        f"sweep_bf16_b1_h16_n8192_d{d}", 1, 16, 8192, d, "bf16", False, 1100 + d,
        note=f"head-width sweep: bf16 N(0,1) inputs, d = {d}, unmasked") for d in (32, 64, 96, 128, 256)},
    "fwd_bf16_b1_h1_n8192_d128": Workload(
        "fwd_bf16_b1_h1_n8192_d128", 1, 1, 8192, 128, "bf16", False, 1201,
        note="one head of the headline shape, bf16 N(0,1) inputs, unmasked"),
    "fwd_bf16_b1_h1_n32768_d128_causal": Workload(
        "fwd_bf16_b1_h1_n32768_d128_causal", 1, 1, 32768, 128, "bf16", True, 1202,
        note="one head of the long-context shape, bf16 N(0,1) inputs, causal"),
    "fwd_bf16_b1_h1_n8192_d128_causal": Workload(
        "fwd_bf16_b1_h1_n8192_d128_causal", 1, 1, 8192, 128, "bf16", True, 1203,
        note="one head of the headline shape, bf16 N(0,1) inputs, causal"),
    "fwd_bf16_b1_h16_n8192_d128_causal": Workload(
        "fwd_bf16_b1_h16_n8192_d128_causal", 1, 16, 8192, 128, "bf16", True, 1204,
        note="the headline shape under the causal mask, bf16 N(0,1) inputs (about the key tiles per CU "
             "of B4 H16 N4096 causal, in half as many workgroups)"),
}
ALL_WORKLOADS = {**WORKLOADS, **EXTRA_WORKLOADS}


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def make(w: Workload, seed: int | None = None) -> dict:
    """Draw q, k, v for workload ``w``.

    Draw order: Q, K, V (float64 normals -> float32 -> storage format), then, for
    the boosted-key workload, the chosen keys of each (b, h) without replacement.
    Returns a dict with arrays ``q``, ``k``, ``v`` of shape [B,H,N,d]: float32 for
    "f32", uint16 bf16 bit patterns for "bf16".

    Boosted keys (a logit offset shared by every query): the last coordinate of
    every query is set to 1 and the last coordinate of every key to 0, except for
    ceil(boost_frac*N) keys per (b, h), whose last coordinate is boost_logit/scale.
    Their scaled score then carries +boost_logit (after bf16 rounding of the
    coordinate: 90.5/sqrt(128) = 7.9991 for d = 128).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape) * w.k_std
    v = rng.standard_normal(shape)
    if w.boost_frac > 0.0:
        nb = int(math.ceil(w.boost_frac * w.N))
        q[..., w.d - 1] = 1.0
        k[..., w.d - 1] = 0.0
        coord = w.boost_logit / w.resolved_scale()
        for b in range(w.B):
            for h in range(w.H):
                idx = rng.choice(w.N, size=nb, replace=False)
                k[b, h, idx, w.d - 1] = coord
    return {"q": _store(q, w.dtype), "k": _store(k, w.dtype), "v": _store(v, w.dtype)}


def make_random(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                q_std: float = 1.0, k_std: float = 1.0, v_std: float = 1.0) -> dict:
    """Generic iid-normal q, k, v of any shape (parity sweeps over shapes and tails)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape) * q_std
    k = rng.standard_normal(shape) * k_std
    v = rng.standard_normal(shape) * v_std
    return {"q": _store(q, dtype), "k": _store(k, dtype), "v": _store(v, dtype)}


def make_backward(B: int, H: int, N: int, d: int, seed: int) -> dict:
    """Seeded bf16 q, k, v and an output gradient dout, all iid N(0,1) (backward checks)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    return {x: _store(rng.standard_normal(shape), "bf16") for x in ("q", "k", "v", "dout")}


def scalar_case(scores, values) -> dict:
    """Express a one-query scalar example through the [B,H,N,d] interface.

    d = 1, scale = 1, every query coordinate is 1 and key j holds score s_j, so
    every query row sees the scores s_j and the value column v_j. Returned as
    float32 arrays of shape [1,1,N,1] (the example's scores must be exact in fp32).
    """
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    n = s.shape[0]
    q = np.ones((1, 1, n, 1), dtype=np.float32)
    k = s.astype(np.float32).reshape(1, 1, n, 1)
    v = vals.astype(np.float32).reshape(1, 1, n, 1)
    if not (np.array_equal(k.astype(np.float64).ravel(), s)
            and np.array_equal(v.astype(np.float64).ravel(), vals)):
        raise ValueError("scalar case values are not exact in float32")
    return {"q": q, "k": k, "v": v}


def sample_rows(N: int, count: int, seed: int, tile_edges=(1, 63, 64, 127, 128, 255, 256)) -> np.ndarray:
    """Query rows for sampled parity at full size: tile edges, the middle, the last
    row, and seeded random rows; max(count, number of fixed rows) unique rows, sorted."""
    fixed = {0, N // 2, N - 1}
    fixed.update(t for t in tile_edges if t < N)
    fixed = np.array(sorted(fixed), dtype=np.int64)
    rest = np.setdiff1d(np.arange(N, dtype=np.int64), fixed)
    rng = np.random.default_rng(seed)
    extra = rng.choice(rest, size=min(len(rest), max(0, count - len(fixed))), replace=False)
    return np.sort(np.concatenate([fixed, extra.astype(np.int64)]))
