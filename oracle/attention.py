"""fp64 CPU oracle for exact dense softmax attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the bench's
CPU-baseline leg may import this module. It shares no code with the HIP path and
imports nothing from it.

What it computes is the plain definition of the operator (lihaoran.work, "The
intermediate matrix comes first": O = softmax(QK^T/sqrt(d)) V, N the sequence
length, d the head dimension), with the caller's score scale in place of
1/sqrt(d) and an optional causal mask (key j kept only when j <= query i). It
materialises the probability matrix one block of query rows at a time, which is
the "standard attention" column of the table in sadullah.online, "Standard
attention vs FlashAttention": scores, then softmax, then the product with V.

Per query row i of each (b, h), in float64:
  s_ij   = scale * sum_c q_ic k_jc            for j in J_i (all j, or j <= i if causal)
  m_i    = max_j s_ij                         (subtracting the max keeps exponents <= 0;
                                               lihaoran.work, "Why averaging block softmaxes fails")
  w_ij   = exp(s_ij - m_i),  l_i = sum_j w_ij
  o_ic   = sum_j w_ij v_jc / l_i
  lse_i  = m_i + ln l_i                       (natural log of the softmax denominator of the
                                               scaled scores; the pages name the running max and
                                               running sum, sadullah.online "Online softmax", and
                                               lse packs both into one number)
The stored inputs are taken exactly: float32 arrays as they are, bf16 arrays as
uint16 bit patterns decoded here.

Parity pins: see tests/test_oracle_pins.py (worked examples from the pages, closed
forms, a library routine, brute-force recurrences, invariants).
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_fp64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input -> float64. ``dtype`` is "bf16" (uint16 bits) or "f32"."""
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _rows_for(rows, b: int, h: int, n: int) -> np.ndarray:
    if rows is None:
        return np.arange(n)
    r = np.asarray(rows)
    return r[b, h] if r.ndim == 3 else r


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, rows=None) -> np.ndarray:
    """Scaled, masked score block for one head: q [N,d], k [N,d] -> s [R,N] (masked = -inf)."""
    n = k.shape[0]
    r = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = scale * (q[r] @ k.T)
    if causal:
        key = np.arange(n)[None, :]
        s = np.where(key > r[:, None], -np.inf, s)
    return s


def probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, rows=None) -> np.ndarray:
    """Softmax of the scaled, masked scores of one head: P [R,N], each row sums to 1."""
    s = scores(q, k, scale, causal, rows)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return w / w.sum(axis=1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
              rows=None, block: int = 512):
    """Exact attention in float64.

    q, k, v: float64 arrays [B,H,N,d] (use ``as_fp64`` on stored inputs).
    rows: None (all query rows), an index array [R] used for every (b, h), or an
    array [B,H,R] of per-head rows.
    Returns (o [B,H,R,d], lse [B,H,R]) as float64.
    """
    B, H, N, d = q.shape
    if k.shape != (B, H, N, d) or v.shape[:3] != (B, H, N):
        raise ValueError("q, k, v shapes disagree")
    dv = v.shape[3]
    r0 = _rows_for(rows, 0, 0, N)
    o = np.empty((B, H, len(r0), dv), dtype=np.float64)
    lse = np.empty((B, H, len(r0)), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            r = _rows_for(rows, b, h, N)
            kb, vb = k[b, h], v[b, h]
            for start in range(0, len(r), block):
                rr = r[start:start + block]
                s = scores(q[b, h], kb, scale, causal, rr)
                m = s.max(axis=1)
                w = np.exp(s - m[:, None])
                l = w.sum(axis=1)
                o[b, h, start:start + len(rr)] = (w @ vb) / l[:, None]
                lse[b, h, start:start + len(rr)] = m + np.log(l)
    return o, lse


def attention_stored(q, k, v, dtype: str, scale: float, causal: bool, rows=None, block: int = 512):
    """``attention`` on stored inputs (float32 arrays or bf16 uint16 bit patterns)."""
    return attention(as_fp64(q, dtype), as_fp64(k, dtype), as_fp64(v, dtype), scale, causal, rows, block)
