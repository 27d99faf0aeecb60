"""Helpers shared by the tests: fp64 views of stored workloads for the oracle."""
import numpy as np

from synth import as_f64


def f64_weights(w, weights):
    """fp64 copy of a stored weight dict (token table excluded)."""
    out = {k: as_f64(v) for k, v in weights.items()
           if k not in ("layers", "tok_emb") and v is not None}
    out["layers"] = [{k: as_f64(v) for k, v in lw.items()} for lw in weights["layers"]]
    return out


def golden(name):
    """Parse a golden fixture: 'key: value' lines, '#' comments ignored."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows
