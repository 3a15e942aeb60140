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
    ("online.py", "factor = 0.0 if m == -math.inf else math.exp(m - m_new)", "factor = 1.0",
     "block merge never rescales"),
    ("online.py", "total = total * factor", "total = total", "block merge rescales only the numerator"),
    ("online.py", "total = rescale * total + w", "total = total + w", "scalar recurrence drops the rescale"),
    ("online.py", "weighted = rescale * weighted + w * val", "weighted = rescale * weighted + val",
     "scalar recurrence drops the weight"),
    ("online.py", "running_sum = running_sum * math.exp(running_max - new_max)",
     "running_sum = running_sum", "normaliser never rescales"),
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
