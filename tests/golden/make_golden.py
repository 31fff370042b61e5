"""Write oracle_regression.json from the oracle alone (no GPU code involved).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.rand(shape, generator=g, dtype=torch.float32) * 2 - 1).numpy()


def main():
    a, b, s = _rand((3, 5), 100), _rand((5, 4), 101), _rand((4,), 102)
    ra = oracle.addmm(a, b, s, False, 0.5, 2.0)
    x, w, bias = _rand((1, 2, 5, 5), 103), _rand((3, 2, 3, 3), 104), _rand((3,), 105)
    rc = oracle.conv2d(x, w, bias, (2, 1), (1, 1), (1, 2))
    out = {
        "addmm": {"seeds": [100, 101, 102], "shape_MKN": [3, 5, 4], "self_2d": False,
                  "beta": 0.5, "alpha": 2.0, "ref": ra.ref.tolist(), "sabs": ra.sabs.tolist()},
        "conv2d": {"seeds": [103, 104, 105], "input": [1, 2, 5, 5], "weight": [3, 2, 3, 3],
                   "stride": [2, 1], "padding": [1, 1], "dilation": [1, 2],
                   "ref": rc.ref.tolist(), "sabs": rc.sabs.tolist()},
        "draw": "torch.Generator('cpu').manual_seed(seed); rand*2-1, fp32",
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    np.set_printoptions(precision=17)
    main()
