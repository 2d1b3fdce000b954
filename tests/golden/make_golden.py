"""Write small_cases.json: small seeded cases evaluated by the fp64 oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import harp_oracle as O  # noqa: E402

CASES = [((2, 3, 2), 0.3), ((5, 2), 0.2), ((4, 3), 0.1), ((8, 2), 0.5), ((3, 3, 2), 0.05)]


def main():
    rng = np.random.default_rng(777)
    out = []
    for sch, sigma in CASES:
        d = int(np.prod(sch))
        theta = rng.standard_normal(sum(O.theta_counts(sch, d))) * sigma
        gauss = np.concatenate([rng.standard_normal(b * b) for b in sch if not O.is_pow2(b)] or [np.zeros(0)])
        signs = np.where(rng.integers(0, 2, d) == 1, 1, -1)
        x = rng.standard_normal((3, d))
        blocks = O.materialize_blocks(sch, d, theta, gauss)
        y = O.apply(x, sch, blocks, signs.astype(float))
        out.append({"schedule": list(sch), "d": d, "theta": theta.tolist(), "gauss": gauss.tolist(),
                    "signs": signs.tolist(), "x": x.tolist(), "y": y.tolist()})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "small_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
