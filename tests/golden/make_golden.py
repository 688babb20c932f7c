"""Write the oracle regression fixtures in this folder.  Calls only ``oracle/`` and the
seeded input generators.

The pages print no worked example of the spectral layer, so these fixtures are not pins:
they freeze the oracle's current output on tiny seeded cases so that any later change to
its arithmetic shows up as a failing test (and must then be justified by the passage, or
the reading of it, that requires the change).

Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle.fno_oracle as O  # noqa: E402
from fno_spectral_convolution_amd import inputs  # noqa: E402

CASES = [
    {"name": "block2d_8x8", "seed": 1, "batch": 1, "cin": 2, "cout": 2, "grid": [8, 8],
     "modes": [3, 3], "tanh": False},
    {"name": "block3d_4x4x6_tanh", "seed": 2, "batch": 1, "cin": 2, "cout": 3,
     "grid": [4, 4, 6], "modes": [1, 2, 2], "tanh": True},
]


def compute(case):
    x, w, wb, b = inputs.small_case(case["seed"], case["batch"], case["cin"], case["cout"],
                                    case["grid"], case["modes"])
    gy = inputs.normal_like(case["seed"], (case["batch"], case["cout"]) + tuple(case["grid"]))
    fwd = O.block_fwd(x, w, wb, b, case["modes"], tanh=case["tanh"])
    bwd = O.block_bwd(x, w, wb, b, case["modes"], gy, tanh=case["tanh"])
    return {
        "y": fwd["y"].ravel().tolist(),
        "y_spec": fwd["y_spec"].ravel().tolist(),
        "grad_x": bwd["grad_x"].ravel().tolist(),
        "grad_w_re": np.real(bwd["grad_w"]).ravel().tolist(),
        "grad_w_im": np.imag(bwd["grad_w"]).ravel().tolist(),
        "grad_wb": bwd["grad_wb"].ravel().tolist(),
        "grad_bias": bwd["grad_bias"].ravel().tolist(),
    }


def main():
    for case in CASES:
        rec = dict(case)
        rec["written_by"] = "tests/golden/make_golden.py (oracle only)"
        rec["values"] = compute(case)
        with open(os.path.join(HERE, case["name"] + ".json"), "w") as f:
            json.dump(rec, f, indent=0)


if __name__ == "__main__":
    main()
