"""The battery of pins that ties the CPU oracle's gradients (oracle.backward) to facts
outside itself.

Each pin is a function ``pin_x(att, bwd)`` taking the forward oracle module
(``oracle.attention``) and the backward module (``oracle.backward``, or a mutated
copy) and raising on failure. ``run_all`` returns the names of the pins that fail.

Sources of truth used here, none of them the gradient code itself:
* central finite differences of the forward oracle (brute force on tiny inputs);
* a library routine: torch's float64 autograd through scaled_dot_product_attention;
* closed forms for special inputs, derived by hand next to each pin;
* invariants of the softmax Jacobian.
"""
from __future__ import annotations

import numpy as np


def _rand(seed, B, H, N, d):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(4)]


def _loss(att, q, k, v, do, scale, causal):
    o, _ = att.attention(q, k, v, scale, causal)
    return float((o * do).sum())


def pin_finite_differences(att, bwd):
    """Central differences of L = sum(dO * O) match the gradients on a tiny problem."""
    for causal in (False, True):
        q, k, v, do = _rand(11 + causal, 1, 2, 6, 3)
        scale, h = 0.7, 1e-5
        dq, dk, dv = bwd.gradients(q, k, v, do, scale, causal)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = _loss(att, q, k, v, do, scale, causal)
                x[idx] = old - h
                lm = _loss(att, q, k, v, do, scale, causal)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            assert np.max(np.abs(num - g)) < 1e-7, np.max(np.abs(num - g))


def pin_library_autograd(att, bwd):
    """torch's float64 autograd through its own attention routine gives the same gradients."""
    import torch
    for causal in (False, True):
        q, k, v, do = _rand(21 + causal, 2, 2, 17, 5)
        scale = 0.45
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        o.backward(torch.tensor(do))
        dq, dk, dv = bwd.gradients(q, k, v, do, scale, causal)
        for g, t in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.max(np.abs(g - t.grad.numpy())) < 1e-12


def pin_constant_values(att, bwd):
    """All values equal: O does not depend on P, so dQ = dK = 0 exactly up to rounding,
    and dV = P^T dO still distributes dO over the keys (sum over keys = sum of dO)."""
    q, k, _, do = _rand(31, 1, 1, 9, 4)
    v = np.broadcast_to(np.array([0.3, -1.2, 2.0, 0.5]), (1, 1, 9, 4)).copy()
    for causal in (False, True):
        dq, dk, dv = bwd.gradients(q, k, v, do, 0.6, causal)
        assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
        # each row of P sums to 1, so the key-sum of dV is the query-sum of dO
        assert np.allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-12)


def pin_zero_queries(att, bwd):
    """q = 0: every visible key has the same weight. Unmasked: dV_j = (1/N) sum_i dO_i.
    Causal: row i weighs keys 0..i by 1/(i+1), so dV_j = sum_{i >= j} dO_i / (i+1)."""
    _, k, v, do = _rand(41, 1, 2, 7, 3)
    q = np.zeros_like(k)
    n = 7
    _, _, dv = bwd.gradients(q, k, v, do, 1.3, False)
    assert np.allclose(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape), rtol=0, atol=1e-13)
    _, _, dv = bwd.gradients(q, k, v, do, 1.3, True)
    expect = np.zeros_like(dv)
    for j in range(n):
        for i in range(j, n):
            expect[:, :, j] += do[:, :, i] / (i + 1)
    assert np.allclose(dv, expect, rtol=0, atol=1e-13)


def pin_key_shift(att, bwd):
    """Adding one vector c to every key shifts all visible scores of row i by scale q_i.c,
    which the softmax ignores: P, dS and therefore dQ and dK are unchanged."""
    q, k, v, do = _rand(51, 1, 2, 8, 4)
    c = np.array([0.7, -2.0, 1.1, 0.4])
    for causal in (False, True):
        g0 = bwd.gradients(q, k, v, do, 0.8, causal)
        g1 = bwd.gradients(q, k + c, v, do, 0.8, causal)
        for a, b in zip(g0, g1):
            assert np.allclose(a, b, rtol=0, atol=1e-11)


def pin_key_gradient_sum(att, bwd):
    """Each row of dS sums to zero (the softmax Jacobian annihilates constants), so the
    gradients of all keys sum to zero: sum_j dK_j = scale sum_i q_i sum_j dS_ij = 0."""
    q, k, v, do = _rand(61, 2, 1, 11, 3)
    for causal in (False, True):
        _, dk, _ = bwd.gradients(q, k, v, do, 0.9, causal)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12


def pin_delta_identity(att, bwd):
    """sum_c dO_ic O_ic (what a kernel computes from its saved output) equals
    sum_k P_ik dP_ik (the Jacobian's row term), because O_i = sum_k P_ik v_k."""
    q, k, v, do = _rand(71, 1, 2, 10, 4)
    for causal in (False, True):
        o, _ = att.attention(q, k, v, 0.5, causal)
        dl = bwd.delta(o, do)
        for h in range(2):
            p = att.probabilities(q[0, h], k[0, h], 0.5, causal)
            dp = do[0, h] @ v[0, h].T
            assert np.allclose(dl[0, h], (p * dp).sum(axis=1), rtol=0, atol=1e-13)


def pin_sampled_matches_full(att, bwd):
    """gradients_sampled (dQ rows from their own rows of P; dK and dV rows from the columns of P
    and dS, built from the forward's lse and the delta identity) equals the full gradients on
    the selected rows, both masks."""
    q, k, v, do = _rand(81, 2, 2, 37, 5)
    qr = np.array([0, 5, 17, 36])
    kr = np.array([0, 1, 20, 36])
    for causal in (False, True):
        dq, dk, dv = bwd.gradients(q, k, v, do, 0.7, causal)
        sq, sk, sv = bwd.gradients_sampled(q, k, v, do, 0.7, causal, qr, kr)
        assert np.allclose(sq, dq[:, :, qr], rtol=0, atol=1e-12)
        assert np.allclose(sk, dk[:, :, kr], rtol=0, atol=1e-12)
        assert np.allclose(sv, dv[:, :, kr], rtol=0, atol=1e-12)


PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}


def run_all(att, bwd):
    """Names of the pins that fail (an exception counts as a failure)."""
    failed = []
    for name, fn in PINS.items():
        try:
            fn(att, bwd)
        except Exception:  # noqa: BLE001 - any exception is a caught mistake
            failed.append(name)
    return failed
