"""The pages' online-softmax recurrences, in plain Python float64.

TEST INFRASTRUCTURE ONLY (same rule as oracle.attention: tests, the smoke check and
the bench's CPU-baseline leg may use it; it shares nothing with the HIP path).

These are the small, slow forms of the algorithm the kernel runs. They serve as
brute-force checks of the materialised oracle in oracle.attention: a mistake in
either one shows up as a disagreement between the two.

* ``online_scalar``: one score at a time (lihaoran.work, "Why averaging block
  softmaxes fails": carry a running max m, an unnormalised total l and a weighted
  sum u; when a new score a arrives, m' = max(m, a), both l and u are multiplied by
  exp(m - m') and the new term enters with weight exp(a - m'); the output is u / l).
* ``merge_block``: one block of scores with vector values (interactiveml.org,
  "FlashAttention saves the matrix...": three sufficient statistics, one rescale
  factor applied to everything accumulated so far, which is 0 while nothing has
  been accumulated, i.e. while m is -inf). Also the update equations of
  liminalml.com "FlashAttention": m' = max(m, max s), a = e^(m-m'), p = e^(s-m'),
  l' = a l + sum p, u' = a u + p V, and after the last block the output u / l.
* ``online_blocks``: ``merge_block`` over consecutive blocks of one score row.
* ``normaliser_blocks``: running max and running sum only (sadullah.online,
  "Online softmax: the algorithmic key").
* ``tiled_attention``: the whole operator on [B,H,N,d] arrays, one query row at a
  time, keys consumed in blocks through ``merge_block``.
* ``block_average``: the wrong method (average of per-block softmax outputs), kept
  only so a test can show it differs (lihaoran.work, "Why averaging block softmaxes
  fails": the block denominators differ).
"""
from __future__ import annotations

import math


def online_scalar(scores, values):
    m, total, weighted = -math.inf, 0.0, 0.0
    for a, val in zip(scores, values):
        m_new = max(m, a)
        rescale = math.exp(m - m_new)          # exp(-inf) = 0 for the first element
        w = math.exp(a - m_new)
        total = rescale * total + w
        weighted = rescale * weighted + w * val
        m = m_new
    return weighted / total


def merge_block(block_scores, block_values, m, total, acc):
    """One online step. block_values: list of value vectors (lists), acc: list.

    Returns the new (m, total, acc). A block whose scores are all -inf leaves the
    state unchanged.
    """
    m_new = max(m, max(block_scores))
    if m_new == -math.inf:
        return m, total, acc
    factor = 0.0 if m == -math.inf else math.exp(m - m_new)
    total = total * factor
    acc = [x * factor for x in acc]
    for s, vec in zip(block_scores, block_values):
        w = math.exp(s - m_new)
        total += w
        acc = [x + w * y for x, y in zip(acc, vec)]
    return m_new, total, acc


def online_blocks(scores, values, block):
    """Blocked online softmax-weighted sum of one score row with scalar values.

    Returns (output, m, total) with output = acc / total.
    """
    m, total, acc = -math.inf, 0.0, [0.0]
    for start in range(0, len(scores), block):
        m, total, acc = merge_block(scores[start:start + block],
                                    [[x] for x in values[start:start + block]], m, total, acc)
    return acc[0] / total, m, total


def normaliser_blocks(blocks):
    """Running (max, sum of exp(s - max)) over a sequence of score blocks."""
    running_max, running_sum = -math.inf, 0.0
    for blk in blocks:
        new_max = max(running_max, max(blk))
        running_sum = running_sum * math.exp(running_max - new_max) + sum(math.exp(s - new_max) for s in blk)
        running_max = new_max
    return running_max, running_sum


def tiled_attention(q, k, v, scale, causal, block=64):
    """Whole operator, row by row, keys merged in blocks. q,k,v: nested [B][H][N][d]
    sequences of floats (numpy arrays work). Returns (o, lse) as nested lists.

    Pure-Python loops: small inputs only.
    """
    B, H, N = len(q), len(q[0]), len(q[0][0])
    o = [[[None] * N for _ in range(H)] for _ in range(B)]
    lse = [[[None] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            qs, ks, vs = q[b][h], k[b][h], v[b][h]
            for i in range(N):
                n_keys = i + 1 if causal else N
                row = [scale * sum(float(x) * float(y) for x, y in zip(qs[i], ks[j])) for j in range(n_keys)]
                vals = [[float(x) for x in vs[j]] for j in range(n_keys)]
                m, total, acc = -math.inf, 0.0, [0.0] * len(vals[0])
                for start in range(0, n_keys, block):
                    m, total, acc = merge_block(row[start:start + block], vals[start:start + block], m, total, acc)
                o[b][h][i] = [x / total for x in acc]
                lse[b][h][i] = m + math.log(total)
    return o, lse


def block_average(scores, values, block):
    """Average of per-block softmax-weighted sums (NOT attention; a counterexample)."""
    outs = []
    for start in range(0, len(scores), block):
        s = scores[start:start + block]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        outs.append(sum(a * b for a, b in zip(w, values[start:start + block])) / sum(w))
    return sum(outs) / len(outs)
