"""The per-row fp32 bound of the GPU parity tests (tests/gpu_util.py::fp32_row_tolerance) against
its closed form on small hand-made inputs: u * max|v| * (1 + L_r), L_r = |scale| log2(e)
max over visible keys of sum_i |q_i k_ji|, u = 2^-24."""
import math

import numpy as np

from gpu_util import fp32_row_tolerance

U = 2.0 ** -24


def _case():
    q = np.array([[[[1.0, -2.0], [0.5, 0.0], [-3.0, 1.0]]]], dtype=np.float32)
    k = np.array([[[[2.0, 1.0], [-1.0, 4.0], [0.0, -0.5]]]], dtype=np.float32)
    v = np.array([[[[0.5, -6.0], [1.0, 2.0], [3.0, 0.25]]]], dtype=np.float32)
    return {"q": q, "k": k, "v": v}


def test_row_bound_closed_form_unmasked():
    t = _case()
    # sum_i |q_i k_ji| per (query, key): rows of |q| times columns of |k|^T
    A = np.array([[4.0, 9.0, 1.0], [1.0, 0.5, 0.0], [7.0, 7.0, 0.5]])
    L = 0.7 * math.log2(math.e) * A.max(1)
    got = fp32_row_tolerance(t, -0.7, False)["row"][0, 0]
    assert np.allclose(got, U * 6.0 * (1.0 + L), rtol=1e-12, atol=0)


def test_row_bound_causal_sees_only_earlier_keys():
    t = _case()
    # query 1 sees keys 0 and 1 only (|q1|.|k0| = 1, |q1|.|k1| = 0.5); query 0 sees key 0
    L = 0.7 * math.log2(math.e) * np.array([4.0, 1.0, 7.0])
    got = fp32_row_tolerance(t, 0.7, True)["row"][0, 0]
    assert np.allclose(got, U * 6.0 * (1.0 + L), rtol=1e-12, atol=0)


def test_row_bound_at_zero_scale_is_the_roundoff_floor():
    got = fp32_row_tolerance(_case(), 0.0, False)["row"]
    assert np.allclose(got, U * 6.0, rtol=1e-12, atol=0)
