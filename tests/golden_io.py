"""Reader of the hand-worked fixtures under tests/golden/.

A fixture is text: '#' comments, then lines 'name token token ...'.  A token is a
number or an expression over numbers, ln (the natural log) and inf; it is evaluated
with nothing else in scope.  Shapes come from the S, H, KV, d lines.
"""
import math
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_SHAPES = {"Q": "SHd", "dO": "SHd", "O": "SHd", "dQ": "SHd",
           "K": "SKd", "V": "SKd", "dK": "SKd", "dV": "SKd",
           "LSE": "SH", "seg": "S"}


def _value(tok):
    return float(eval(tok, {"__builtins__": {}}, {"ln": math.log, "inf": math.inf}))


def golden_files():
    return sorted(os.path.join(GOLDEN_DIR, f) for f in os.listdir(GOLDEN_DIR)
                  if f.endswith(".txt"))


def load_golden(path):
    """Returns a dict: ints S, H, KV, d; float scale; float64 arrays for the
    tensors (seg as uint32), shaped as the fixture's header says."""
    raw = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                raw[line[0]] = line[1:]
    out = {k: int(raw[k][0]) for k in ("S", "H", "KV", "d")}
    out["scale"] = _value(raw["scale"][0])
    dims = {"S": out["S"], "H": out["H"], "K": out["KV"], "d": out["d"]}
    for name, shape in _SHAPES.items():
        vals = np.array([_value(t) for t in raw[name]], np.float64)
        out[name] = vals.reshape([dims[c] for c in shape])
    out["seg"] = out["seg"].astype(np.uint32)
    return out


def pad_head_dim(g, d):
    """The same problem with the head dimension zero-padded to d: every dot
    product is unchanged, so the padded gradients are the fixture's in column 0
    and zero elsewhere."""
    p = dict(g)
    for name in ("Q", "dO", "O", "dQ", "K", "V", "dK", "dV"):
        a = np.zeros(g[name].shape[:-1] + (d,), np.float64)
        a[..., :g["d"]] = g[name]
        p[name] = a
    p["d"] = d
    return p
