"""Write the stored expected values under tests/golden/ (calls only oracle/).

    python tests/golden/make_golden.py

Each file holds the codec tables the oracle derives for one (d, bits, seed)
and a small encode example with its inputs.  Floats are stored as exact
hexadecimal strings (float.hex) so nothing is lost in JSON.
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle as O  # noqa: E402


def hexlist(a):
    return [float(x).hex() for x in np.asarray(a, dtype=np.float64).ravel()]


def codec_file(d, bits, seed):
    cd = O.make_codec(d, bits, seed=seed)
    S = np.ascontiguousarray(cd.S, dtype=np.float32)
    rec = {
        "d": d, "bits": bits, "m": cd.m, "seed": seed,
        "lloyd_max_iterations": cd.iters,
        "centroids": hexlist(cd.centroids),
        "bounds": hexlist(cd.bounds),
        "D_signs": "".join("+" if v > 0 else "-" for v in cd.D),
        "S_sha256": hashlib.sha256(S.tobytes()).hexdigest(),
        "S_first_row_head": hexlist(S[0, :16]),
        "S_last_row_tail": hexlist(S[-1, -16:]),
    }
    if d <= 256:
        rng = np.random.default_rng(20240000 + d * 10 + bits)
        x = rng.standard_normal((8, d)).astype(np.float32)
        x[3] = 0.0                      # zero vector
        x[5] = 0.0; x[5, 7] = 2.5       # basis vector
        enc = O.encode(cd, x.astype(np.float64))
        rec["example"] = {
            "x_f32": hexlist(x),
            "codes": enc["codes"].astype(np.uint32).tolist(),
            "signs": enc["signs"].astype(np.uint32).tolist(),
            "norm": hexlist(enc["norm"]),
            "rnorm": hexlist(enc["rnorm"]),
            "y": hexlist(enc["y"]),
            "z": hexlist(enc["z"]),
        }
    name = f"codec_d{d}_b{bits}_s{seed}.json"
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", name)


if __name__ == "__main__":
    for d, bits in [(128, 3), (128, 4), (64, 2), (1536, 4), (1536, 3)]:
        codec_file(d, bits, 1234)
