"""The online softmax of the pages, as slow float64 reference code.

TEST INFRASTRUCTURE ONLY (same rule as oracle.attention: tests, the smoke check and
the bench's CPU-baseline leg may use it; it shares nothing with the HIP path).

These are small, slow forms of the algorithm the kernels run. They serve as independent
checks of the materialised oracle in oracle.attention, which follows a different route
(the whole score row at once): a mistake in either one shows up as a disagreement.

The construction follows the update equations (liminalml.com, "FlashAttention", online
update equations) and the merge of three sufficient statistics (interactiveml.org,
"FlashAttention saves the matrix, not the quadratic work"). A set of (score, value) pairs
is summarised by a State (m, l, u): m its largest score, l = sum_j e^(s_j - m) and
u = sum_j e^(s_j - m) v_j. Two states merge into the state of their union with
m* = max(m_a, m_b) and each side scaled by e^(m - m*), which is 0 for a side that holds no
pair (m = -inf). The softmax average of a set is u / l and its log-normaliser m + ln l.
Every function below is a fold of ``merge`` over block states:

* ``online_scalar``: one pair at a time (the scalar recurrence of lihaoran.work,
  "Check three scores"), output u / l.
* ``merge_block``: the update of a running state by one block with vector values; the
  block's own state is formed first, then merged.
* ``online_blocks``: consecutive blocks of one score row with scalar values.
* ``normaliser_blocks``: running max and sum only (sadullah.online, "Online softmax: the
  algorithmic key").
* ``tiled_attention``: the whole operator on [B,H,N,d] arrays, one query row at a time,
  keys consumed in blocks.
* ``block_average``: the wrong method (average of per-block softmax outputs), kept only so
  that a test can show that it differs (lihaoran.work, "Why averaging block softmaxes
  fails": the blocks' denominators differ).
"""
from __future__ import annotations

import functools
import math

import numpy as np


class State:
    """Three sufficient statistics of a set of (score, value) pairs: the largest score m, the
    sum l of e^(s - m) and the sum u of e^(s - m) v (a float64 vector)."""

    __slots__ = ("m", "l", "u")

    def __init__(self, m: float, l: float, u: np.ndarray):
        self.m, self.l, self.u = m, l, u


def empty(width: int) -> State:
    return State(-math.inf, 0.0, np.zeros(width))


def block_state(scores, values) -> State:
    """State of one block on its own. values: one value vector per score (or scalars)."""
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64).reshape(len(s), -1)
    m = float(s.max())
    if m == -math.inf:                      # every score masked: the block holds no pair
        return empty(vals.shape[1])
    p = np.exp(s - m)
    return State(m, float(p.sum()), p @ vals)


def merge(a: State, b: State) -> State:
    """State of the union of two sets: each side weighted by e^(m - m*), m* = max(m_a, m_b)."""
    m = max(a.m, b.m)
    if m == -math.inf:
        return State(m, 0.0, np.zeros_like(a.u))
    wa = 0.0 if a.m == -math.inf else math.exp(a.m - m)
    wb = 0.0 if b.m == -math.inf else math.exp(b.m - m)
    return State(m, wa * a.l + wb * b.l, wa * a.u + wb * b.u)


def online_scalar(scores, values) -> float:
    """Softmax-weighted average of scalar values, folding in one pair at a time."""
    st = functools.reduce(merge, (block_state([s], [v]) for s, v in zip(scores, values)), empty(1))
    return float(st.u[0] / st.l)


def merge_block(block_scores, block_values, m, total, acc):
    """Running state (m, total, acc) updated by one block. block_values: list of value vectors,
    acc: list. Returns the new (m, total, acc) as plain floats and a list. A block whose scores
    are all -inf leaves the state unchanged."""
    st = merge(State(m, total, np.asarray(acc, dtype=np.float64)), block_state(block_scores, block_values))
    return st.m, st.l, [float(x) for x in st.u]


def online_blocks(scores, values, block):
    """One score row with scalar values, consumed in blocks of `block`. Returns
    (output, m, total) with output = u / total."""
    st = functools.reduce(
        merge, (block_state(scores[i:i + block], values[i:i + block]) for i in range(0, len(scores), block)),
        empty(1))
    return float(st.u[0] / st.l), st.m, st.l


def normaliser_blocks(blocks):
    """Running (max, sum of e^(s - max)) over a sequence of score blocks."""
    st = functools.reduce(merge, (block_state(b, [0.0] * len(b)) for b in blocks), empty(1))
    return st.m, st.l


def tiled_attention(q, k, v, scale, causal, block=64):
    """Whole operator, row by row, keys merged in blocks. q,k,v: nested [B][H][N][d]
    sequences of floats (numpy arrays work). Returns (o, lse) as nested lists.

    Python loops over rows: small inputs only.
    """
    B, H, N = len(q), len(q[0]), len(q[0][0])
    o = [[[None] * N for _ in range(H)] for _ in range(B)]
    lse = [[[None] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            qs = np.asarray(q[b][h], dtype=np.float64)
            ks = np.asarray(k[b][h], dtype=np.float64)
            vs = np.asarray(v[b][h], dtype=np.float64)
            for i in range(N):
                n_keys = i + 1 if causal else N
                row = [scale * float(np.dot(qs[i], ks[j])) for j in range(n_keys)]
                st = empty(vs.shape[1])
                for start in range(0, n_keys, block):
                    st = merge(st, block_state(row[start:start + block], vs[start:min(start + block, n_keys)]))
                o[b][h][i] = [float(x) for x in st.u / st.l]
                lse[b][h][i] = st.m + math.log(st.l)
    return o, lse


def block_average(scores, values, block):
    """Average of per-block softmax-weighted sums (NOT attention; a counterexample)."""
    outs = []
    for start in range(0, len(scores), block):
        st = block_state(scores[start:start + block], values[start:start + block])
        outs.append(float(st.u[0] / st.l))
    return sum(outs) / len(outs)
