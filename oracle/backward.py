"""fp64 CPU oracle for the gradients of exact softmax attention (the backward pass).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the bench's
CPU-baseline leg may import this module. It shares no code with the HIP path and
imports nothing from it.

The pages mention the backward pass only through what FlashAttention does there:
it recomputes selected quantities instead of storing them (lihaoran.work, "The
intermediate matrix comes first"). The gradients themselves follow from
differentiating the operator's definition (same page and section:
O = softmax(QK^T / sqrt(d)) V, here with the caller's scale and optional causal
mask). With S = scale * Q K^T (masked entries -inf), P = softmax(S) row by row,
O = P V, and dO the gradient of a scalar loss with respect to O, per (b, h):

    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)     (the softmax Jacobian applied to dP)
    dQ = scale * dS K
    dK = scale * dS^T Q

Everything is float64 and P is materialised one block of query rows at a time.
``gradients_sampled`` gives selected rows of the same gradients for full-size inputs (a dK or
dV row needs one column of P and dS, built from the forward's lse and the delta identity).
Parity pins: tests/oracle_bwd_pins.py (central finite differences on tiny inputs, a library
autograd routine in float64, closed forms for special inputs, invariants, and the sampled
entries against the full gradients).
"""
from __future__ import annotations

import numpy as np

from .attention import attention, probabilities


def gradients(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
              causal: bool, block: int = 512):
    """Gradients of sum(dO * O) with respect to q, k, v, all float64 [B,H,N,d].

    Returns (dq, dk, dv) as float64 arrays of the input shapes.
    """
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape[:3] != (B, H, N) or do.shape != v.shape:
        raise ValueError("q, k, v, do shapes disagree")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            qb, kb, vb, dob = q[b, h], k[b, h], v[b, h], do[b, h]
            for start in range(0, N, block):
                rr = np.arange(start, min(N, start + block))
                p = probabilities(qb, kb, scale, causal, rr)          # [R, N], 0 where masked
                dv[b, h] += p.T @ dob[rr]
                dp = dob[rr] @ vb.T                                   # [R, N]
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, rr] = scale * (ds @ kb)
                dk[b, h] += scale * (ds.T @ qb[rr])
    return dq, dk, dv


def delta(o: np.ndarray, do: np.ndarray) -> np.ndarray:
    """Per-row sum_c dO_ic O_ic [B,H,N]: equal to sum_k P_ik dP_ik, since O_i = sum_k P_ik v_k."""
    return (o * do).sum(axis=-1)


def gradients_sampled(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                      causal: bool, q_rows: np.ndarray, k_rows: np.ndarray):
    """Selected entries of the same gradients, for inputs too large for ``gradients``.

    dQ on query rows ``q_rows`` and dK, dV on key rows ``k_rows`` (index arrays used for every
    (b, h)), from the same definitions: a dQ row needs its own row of P and dP; a dK or dV row
    needs the column of P and dS of its key, i.e. P_ij = exp(S_ij - lse_i) and the row term
    delta_i = sum_k P_ik dP_ik = sum_c dO_ic O_ic for every query i, which come from the
    forward oracle (o, lse) over all rows. Returns (dq [B,H,Rq,d], dk [B,H,Rk,d],
    dv [B,H,Rk,d]) in float64.
    """
    B, H, N, d = q.shape
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    o, lse = attention(q, k, v, scale, causal)
    dlt = delta(o, do)
    dq = np.empty((B, H, len(q_rows), d))
    dk = np.empty((B, H, len(k_rows), d))
    dv = np.empty((B, H, len(k_rows), v.shape[3]))
    for b in range(B):
        for h in range(H):
            qb, kb, vb, dob = q[b, h], k[b, h], v[b, h], do[b, h]
            # rows of dQ
            p = probabilities(qb, kb, scale, causal, q_rows)                 # [Rq, N]
            dp = dob[q_rows] @ vb.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ kb)
            # columns of P and dS for the sampled keys, over every query row
            s_cols = scale * (qb @ kb[k_rows].T)                               # [N, Rk]
            if causal:
                s_cols = np.where(k_rows[None, :] > np.arange(N)[:, None], -np.inf, s_cols)
            p_cols = np.exp(s_cols - lse[b, h][:, None])
            dp_cols = dob @ vb[k_rows].T                                       # [N, Rk]
            ds_cols = p_cols * (dp_cols - dlt[b, h][:, None])
            dv[b, h] = p_cols.T @ dob
            dk[b, h] = scale * (ds_cols.T @ qb)
    return dq, dk, dv
