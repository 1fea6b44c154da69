"""The oracle still reproduces its stored tables (regression of tests/golden/,
which tests/golden/make_golden.py writes from the oracle alone)."""
import glob
import hashlib
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "codec_*.json")))


def _f(lst):
    return np.array([float.fromhex(s) for s in lst])


@pytest.mark.parametrize("path", GOLD, ids=[os.path.basename(p) for p in GOLD])
def test_oracle_matches_golden(path):
    g = json.load(open(path))
    cd = O.make_codec(g["d"], g["bits"], seed=g["seed"])
    assert np.array_equal(cd.centroids, _f(g["centroids"]))
    assert np.array_equal(cd.bounds, _f(g["bounds"]))
    assert "".join("+" if v > 0 else "-" for v in cd.D) == g["D_signs"]
    assert hashlib.sha256(np.ascontiguousarray(cd.S).tobytes()).hexdigest() == g["S_sha256"]
    if "example" in g:
        ex = g["example"]
        x = _f(ex["x_f32"]).reshape(-1, g["d"])
        enc = O.encode(cd, x)
        assert np.array_equal(enc["codes"], np.array(ex["codes"], dtype=np.uint32))
        assert np.array_equal(enc["signs"], np.array(ex["signs"], dtype=np.uint32))
        assert np.array_equal(enc["norm"].astype(np.float64), _f(ex["norm"]))
        assert np.array_equal(enc["rnorm"].astype(np.float64), _f(ex["rnorm"]))
