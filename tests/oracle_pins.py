"""The battery of pins that ties the CPU oracle to facts outside itself.

Each pin is a function ``pin_x(att, onl)`` taking the oracle's two modules
(``oracle.attention`` and ``oracle.online``, or mutated copies of them) and raising
AssertionError (or any exception) when the pin fails. ``run_all`` returns the names
of the pins that fail. test_oracle_pins.py requires an empty list for the real
oracle; test_oracle_mutants.py plants plausible mistakes in copies of the oracle and
requires each one to be caught.

Sources of truth used here, none of them the oracle itself:
* worked examples printed on the pages (tests/golden/pages_examples.json);
* closed forms derived by hand (written out next to each pin);
* a library routine: torch's CPU scaled_dot_product_attention in float64;
* the bf16 format definition (a bf16 value is the upper 16 bits of a binary32);
* brute-force recurrences from the pages (oracle.online), which follow a different
  algorithm from the materialised oracle;
* invariants of softmax attention.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))


def _scalar(att, scores, values, causal=False):
    """Run the oracle's [B,H,N,d] attention on a scalar example (d = 1, q = 1, k_j = s_j)."""
    n = len(scores)
    q = np.ones((1, 1, n, 1))
    k = np.asarray(scores, dtype=np.float64).reshape(1, 1, n, 1)
    v = np.asarray(values, dtype=np.float64).reshape(1, 1, n, 1)
    o, lse = att.attention(q, k, v, 1.0, causal)
    return o[0, 0, :, 0], lse[0, 0]


def pin_three_scores(att, onl):
    g = GOLDEN["three_scores"]
    o, _ = _scalar(att, g["scores"], g["values"])
    assert np.all(np.round(o, 6) == g["printed_round6"]), o
    ref = onl.online_scalar(g["scores"], g["values"])
    assert math.isclose(ref, o[0], rel_tol=g["page_rel_tol"])
    # closed form: (10 + 20e + 30e^2) / (1 + e + e^2)
    e = math.e
    assert math.isclose(o[0], (10 + 20 * e + 30 * e * e) / (1 + e + e * e), rel_tol=1e-14)


def pin_shift(att, onl):
    g3, gs = GOLDEN["three_scores"], GOLDEN["shift"]
    base, lse0 = _scalar(att, g3["scores"], g3["values"])
    shifted, lse1 = _scalar(att, [s + gs["offset"] for s in g3["scores"]], g3["values"])
    assert np.allclose(shifted, base, rtol=1e-12, atol=0)
    # softmax is shift invariant; the log-normaliser moves by exactly the shift
    assert np.allclose(lse1 - lse0, gs["offset"], rtol=0, atol=1e-9)
    # closed form of the log-normaliser: ln(1 + e + e^2)
    assert math.isclose(lse0[0], math.log(1 + math.e + math.e ** 2), rel_tol=1e-14)
    assert math.isclose(onl.online_scalar([s + gs["offset"] for s in g3["scores"]], g3["values"]),
                        base[0], rel_tol=g3["page_rel_tol"])


def pin_block_example(att, onl):
    g = GOLDEN["block_example"]
    o, lse = _scalar(att, g["scores"], g["values"])
    # exp(1 - 1002) and exp(2 - 1002) underflow to 0 in float64, so the result is
    # the two-term softmax over scores 1001, 1002: (4 e^-1 + 8) / (e^-1 + 1).
    closed = (4 * math.exp(-1) + 8) / (math.exp(-1) + 1)
    assert abs(o[0] - closed) < g["page_abs_tol"]
    online, m, total = onl.online_blocks(g["scores"], g["values"], g["block"])
    assert abs(online - o[0]) < g["page_abs_tol"]
    assert m == 1002.0
    assert math.isclose(lse[0], 1002.0 + math.log(1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(m + math.log(total), lse[0], rel_tol=1e-15)


def pin_normaliser_blocks(att, onl):
    from scipy.special import logsumexp
    blocks = GOLDEN["normaliser_blocks"]["blocks"]
    flat = [s for b in blocks for s in b]
    m, s = onl.normaliser_blocks(blocks)
    assert m == 4.1
    ref = float(logsumexp(flat))
    assert math.isclose(m + math.log(s), ref, rel_tol=1e-14)
    _, lse = _scalar(att, flat, [0.0] * len(flat))
    assert math.isclose(lse[0], ref, rel_tol=1e-14)


def pin_quiz(att, onl):
    g = GOLDEN["quiz"]
    t0, a0, v_new = 2.5, -0.75, 3.0
    m, total, acc = onl.merge_block([g["new_max"]], [[v_new]], g["old_max"], t0, [a0])
    f = math.exp(g["old_max"] - g["new_max"])
    assert math.isclose(f, math.exp(-5))
    assert m == g["new_max"]
    assert math.isclose(total, f * t0 + 1.0, rel_tol=1e-15)
    assert math.isclose(acc[0], f * a0 + v_new, rel_tol=1e-15)
    # the same state through the scalar recurrence, first score at the old max
    o = onl.online_scalar([g["old_max"], g["new_max"]], [1.0, v_new])
    assert math.isclose(o, (f * 1.0 + v_new) / (f + 1.0), rel_tol=1e-14)


def pin_random_cases(att, onl):
    g = GOLDEN["random_cases"]
    rng = np.random.default_rng(390)
    per = g["count"] // (g["max_len"] - g["min_len"] + 1)
    for length in range(g["min_len"], g["max_len"] + 1):
        for _ in range(per):
            s = rng.normal(0.0, 5.0, length)
            v = rng.normal(0.0, 1.0, length)
            o, _ = _scalar(att, s.tolist(), v.tolist())
            ref = onl.online_scalar(s.tolist(), v.tolist())
            assert math.isclose(o[0], ref, rel_tol=1e-12, abs_tol=1e-12), (length, o[0], ref)
            blk, _, _ = onl.online_blocks(s.tolist(), v.tolist(), 4)
            assert math.isclose(blk, ref, rel_tol=1e-12, abs_tol=1e-12)


def pin_library_sdpa(att, onl):
    """torch's CPU scaled_dot_product_attention in float64, non-square shapes."""
    import torch
    rng = np.random.default_rng(7)
    B, H, N, d, dv = 2, 3, 37, 5, 4
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) * 2.0
    v = rng.standard_normal((B, H, N, dv))
    for causal in (False, True):
        o, lse = att.attention(q, k, v, 0.37, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.37).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-12), (causal, np.abs(o - ref).max())
        # per-head sampled rows agree with the full result
        rows = rng.integers(0, N, size=(B, H, 6))
        o_s, lse_s = att.attention(q, k, v, 0.37, causal, rows=rows)
        for b in range(B):
            for h in range(H):
                assert np.allclose(o_s[b, h], ref[b, h, rows[b, h]], rtol=0, atol=1e-12)
                assert np.allclose(lse_s[b, h], lse[b, h, rows[b, h]], rtol=0, atol=1e-12)


def pin_zero_queries(att, onl):
    """Q = 0: every score is 0, so the weights are uniform over the visible keys.

    o_i = mean of v_j over the visible keys and lse_i = ln(number of visible keys).
    """
    rng = np.random.default_rng(11)
    B, H, N, d = 1, 2, 23, 6
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    o, lse = att.attention(q, k, v, 0.5, False)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-13)
    assert np.allclose(lse, math.log(N), atol=1e-13)
    o, lse = att.attention(q, k, v, 0.5, True)
    counts = np.arange(1, N + 1)
    cummean = np.cumsum(v, axis=2) / counts[None, None, :, None]
    assert np.allclose(o, cummean, atol=1e-13)
    assert np.allclose(lse, np.log(counts)[None, None, :], atol=1e-13)


def pin_causal_first_row(att, onl):
    """Causal row 0 sees only key 0: o_0 = v_0 exactly, lse_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, 9, 4))
    k = rng.standard_normal((1, 1, 9, 4))
    v = rng.standard_normal((1, 1, 9, 4))
    o, lse = att.attention(q, k, v, 0.8, True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert math.isclose(lse[0, 0, 0], 0.8 * float(np.dot(q[0, 0, 0], k[0, 0, 0])), rel_tol=1e-14)


def pin_identity_values(att, onl):
    """V = I (N = d) makes O the probability matrix: rows >= 0 summing to 1."""
    rng = np.random.default_rng(13)
    N = 16
    q = rng.standard_normal((1, 1, N, N))
    k = rng.standard_normal((1, 1, N, N))
    v = np.eye(N).reshape(1, 1, N, N)
    for causal in (False, True):
        o, _ = att.attention(q, k, v, 0.25, causal)
        p = att.probabilities(q[0, 0], k[0, 0], 0.25, causal)
        assert np.allclose(o[0, 0], p, atol=1e-14)
        assert np.all(p >= 0)
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
        if causal:
            assert np.all(np.triu(p, 1) == 0)


def pin_permutations(att, onl):
    """Unmasked: permuting keys with their values changes nothing; permuting queries
    permutes the output rows."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 1, 21, 3))
    k = rng.standard_normal((1, 1, 21, 3))
    v = rng.standard_normal((1, 1, 21, 2))
    o, lse = att.attention(q, k, v, 1.3, False)
    pk = rng.permutation(21)
    o2, lse2 = att.attention(q, k[:, :, pk], v[:, :, pk], 1.3, False)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)
    pq = rng.permutation(21)
    o3, lse3 = att.attention(q[:, :, pq], k, v, 1.3, False)
    assert np.allclose(o3, o[:, :, pq], atol=1e-13) and np.allclose(lse3, lse[:, :, pq], atol=1e-13)


def pin_tiled_online(att, onl):
    """The pages' blocked online algorithm (pure Python) against the materialised oracle."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, 2, 19, 3))
    k = rng.standard_normal((1, 2, 19, 3)) * 3.0
    v = rng.standard_normal((1, 2, 19, 3))
    for causal in (False, True):
        o, lse = att.attention(q, k, v, 0.6, causal)
        ot, lset = onl.tiled_attention(q, k, v, 0.6, causal, block=4)
        assert np.allclose(o, np.array(ot), rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, np.array(lset), rtol=1e-12, atol=1e-12)


def pin_block_average_differs(att, onl):
    g = GOLDEN["block_example"]
    o, _ = _scalar(att, g["scores"], g["values"])
    avg = onl.block_average(g["scores"], g["values"], g["block"])
    assert abs(avg - o[0]) > 1.0


def pin_bf16_decode(att, onl):
    """bf16 is the upper half of a binary32: fixed patterns and every finite pattern
    against torch's own bfloat16 -> float64 conversion."""
    import torch
    fixed = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0000: 0.0, 0x8000: -0.0,
             0x0001: 2.0 ** -133, 0x7F7F: 3.3895313892515355e38, 0x3C00: 2.0 ** -7}
    got = att.decode_bf16(np.array(list(fixed), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(fixed.values())))
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    mine = att.decode_bf16(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(mine[finite], ref[finite])


def pin_stored_inputs(att, onl):
    """attention_stored decodes each storage format and otherwise equals attention."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((1, 1, 5, 2)).astype(np.float32)
    o1, l1 = att.attention_stored(x, x, x, "f32", 0.5, False)
    o2, l2 = att.attention(x.astype(np.float64), x.astype(np.float64), x.astype(np.float64), 0.5, False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    hi = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # truncation: exact bf16 values
    o3, _ = att.attention_stored(hi, hi, hi, "bf16", 0.5, False)
    t = (hi.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    o4, _ = att.attention(t, t, t, 0.5, False)
    assert np.array_equal(o3, o4)


PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}


def run_all(att, onl):
    """Names of the pins that fail (an exception counts as a failure)."""
    failed = []
    for name, fn in PINS.items():
        try:
            fn(att, onl)
        except Exception:  # noqa: BLE001 - any exception is a caught mistake
            failed.append(name)
    return failed
