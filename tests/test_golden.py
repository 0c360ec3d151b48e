"""The oracle reproduces its stored values for the tiny d=16 workload."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _read(path):
    out, cur, rows = {}, None, []
    with open(path) as f:
        for line in f:
            if line.startswith("#"):
                continue
            parts = line.split()
            if len(parts) == 3 and parts[0].isalpha():
                cur = parts[0]
                out[cur] = []
                continue
            out[cur].append([float(x) for x in parts])
    return {k: np.array(v) for k, v in out.items()}


def test_tiny_fixture_matches_oracle():
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden
    stored = _read(os.path.join(HERE, "golden", "tiny_d16_oracle.txt"))
    o, S, y = make_golden.compute()
    for name, arr in (("o", o), ("S", S), ("y", y)):
        assert stored[name].shape == arr.shape
        np.testing.assert_allclose(arr, stored[name], rtol=1e-13, atol=1e-15)
