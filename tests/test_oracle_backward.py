"""The CPU oracle's gradients against finite differences, a library autograd, closed forms
and invariants (pins in oracle_bwd_pins.py), and planted mistakes in copies of
oracle/backward.py that the pins must catch."""
import os
import types

import pytest

import oracle_bwd_pins
from oracle import attention as att
from oracle import backward as bwd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", sorted(oracle_bwd_pins.PINS))
def test_pin(name):
    oracle_bwd_pins.PINS[name](att, bwd)


# (original text, mutated text, what the mistake is)
MUTANTS = [
    ("dq[b, h, rr] = scale * (ds @ kb)", "dq[b, h, rr] = ds @ kb", "scale left out of dQ"),
    ("dk[b, h] += scale * (ds.T @ qb[rr])", "dk[b, h] += scale * (ds.T @ kb[rr])", "keys used for dK"),
    ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp", "row term of the Jacobian dropped"),
    ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
     "ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))", "row term summed over queries"),
    ("dp = dob[rr] @ vb.T", "dp = dob[rr] @ kb.T", "keys used for dP"),
    ("dv[b, h] += p.T @ dob[rr]", "dv[b, h] += p.T @ qb[rr]", "queries used for dV"),
    ("p = probabilities(qb, kb, scale, causal, rr)", "p = probabilities(qb, kb, scale, False, rr)",
     "mask ignored"),
    ("return (o * do).sum(axis=-1)", "return (o * do).sum(axis=-2)", "delta summed over rows"),
    ("ds_cols = p_cols * (dp_cols - dlt[b, h][:, None])", "ds_cols = p_cols * dp_cols",
     "sampled dK: row term dropped"),
    ("p_cols = np.exp(s_cols - lse[b, h][:, None])", "p_cols = np.exp(s_cols)", "sampled columns: lse not subtracted"),
    ("s_cols = np.where(k_rows[None, :] > np.arange(N)[:, None], -np.inf, s_cols)",
     "s_cols = np.where(k_rows[None, :] < np.arange(N)[:, None], -np.inf, s_cols)", "sampled columns: mask reversed"),
]


def _load(src):
    mod = types.ModuleType("bwd_m")
    mod.__file__ = os.path.join(ROOT, "oracle", "backward.py")
    mod.__dict__["probabilities"] = att.probabilities
    mod.__dict__["attention"] = att.attention
    src = src.replace("from .attention import attention, probabilities\n", "")
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes():
    src = open(os.path.join(ROOT, "oracle", "backward.py")).read()
    assert oracle_bwd_pins.run_all(att, _load(src)) == []


@pytest.mark.parametrize("mutation", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_mutant_is_caught(mutation):
    old, new, what = mutation
    src = open(os.path.join(ROOT, "oracle", "backward.py")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    failed = oracle_bwd_pins.run_all(att, _load(src.replace(old, new)))
    assert failed, f"no pin caught: {what}"
