"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the
pin battery catches every one of them. This shows the pins constrain each part of
the oracle: the score product and its scale, the mask, the max subtraction, the
normalisation, the log-normaliser, the bf16 decode and the online recurrences."""
import importlib.util
import os
import types

import pytest

import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (file, original text, mutated text, what the mistake is)
MUTANTS = [
    ("attention.py", "s = scale * (q[r] @ k.T)", "s = (q[r] @ k.T)", "score scale dropped"),
    ("attention.py", "s = scale * (q[r] @ k.T)", "s = scale * (k[r] @ q.T)", "q and k swapped"),
    ("attention.py", "key > r[:, None]", "key >= r[:, None]", "mask hides the diagonal"),
    ("attention.py", "key > r[:, None]", "key < r[:, None]", "mask reversed"),
    ("attention.py", "key > r[:, None]", "key > r[:, None] + 1", "mask lets one future key in"),
    ("attention.py", "w = np.exp(s - m[:, None])", "w = np.exp(s)", "max not subtracted"),
    ("attention.py", "o[b, h, start:start + len(rr)] = (w @ vb) / l[:, None]",
     "o[b, h, start:start + len(rr)] = (w @ vb)", "output not normalised"),
    ("attention.py", "o[b, h, start:start + len(rr)] = (w @ vb) / l[:, None]",
     "o[b, h, start:start + len(rr)] = (w @ kb[:, :vb.shape[1]]) / l[:, None]", "k used as values"),
    ("attention.py", "lse[b, h, start:start + len(rr)] = m + np.log(l)",
     "lse[b, h, start:start + len(rr)] = np.log(l)", "max left out of lse"),
    ("attention.py", "lse[b, h, start:start + len(rr)] = m + np.log(l)",
     "lse[b, h, start:start + len(rr)] = m + np.log2(l)", "wrong log base"),
    ("attention.py", "l = w.sum(axis=1)\n", "l = w.sum(axis=1) + 1e-9\n", "stray term in the denominator"),
    ("attention.py", "<< np.uint32(16)", "<< np.uint32(15)", "bf16 decode shifted"),
    ("attention.py", "kb, vb = k[b, h], v[b, h]", "kb, vb = k[b, 0], v[b, h]", "wrong head index for k"),
    ("attention.py", "r = _rows_for(rows, b, h, N)", "r = _rows_for(rows, 0, 0, N)", "per-head rows ignored"),
    ("attention.py", "return w / w.sum(axis=1, keepdims=True)", "return w / w.sum(axis=0, keepdims=True)",
     "probabilities normalised over queries"),
    ("online.py", "wa = 0.0 if a.m == -math.inf else math.exp(a.m - m)", "wa = 0.0 if a.m == -math.inf else 1.0",
     "merge never rescales the running side"),
    ("online.py", "wb = 0.0 if b.m == -math.inf else math.exp(b.m - m)", "wb = 1.0",
     "merge never rescales the incoming block"),
    ("online.py", "return State(m, wa * a.l + wb * b.l, wa * a.u + wb * b.u)",
     "return State(m, a.l + wb * b.l, wa * a.u + wb * b.u)", "merge rescales only the numerator"),
    ("online.py", "m = max(a.m, b.m)", "m = min(a.m, b.m)", "merge keeps the smaller max"),
    ("online.py", "p = np.exp(s - m)", "p = np.exp(s)", "block state without the max subtraction"),
    ("online.py", "return State(m, float(p.sum()), p @ vals)", "return State(m, float(p.sum()), vals.sum(axis=0))",
     "block state drops the weights of the values"),
]


def _load(fname, src, name):
    mod = types.ModuleType(name)
    mod.__file__ = os.path.join(ROOT, "oracle", fname)
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


def _modules(mutation=None):
    srcs = {f: open(os.path.join(ROOT, "oracle", f)).read() for f in ("attention.py", "online.py")}
    if mutation is not None:
        fname, old, new, _ = mutation
        assert srcs[fname].count(old) >= 1, f"mutation anchor not found in {fname}: {old!r}"
        srcs[fname] = srcs[fname].replace(old, new)
    return _load("attention.py", srcs["attention.py"], "att_m"), _load("online.py", srcs["online.py"], "onl_m")


def test_unmutated_copy_passes():
    att, onl = _modules()
    assert oracle_pins.run_all(att, onl) == []


@pytest.mark.parametrize("mutation", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_mutant_is_caught(mutation):
    att, onl = _modules(mutation)
    failed = oracle_pins.run_all(att, onl)
    assert failed, f"no pin caught: {mutation[3]}"
