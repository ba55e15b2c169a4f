"""Write tests/golden/brute_force_cases.json.

Calls only the oracle's exact rational brute force on the seeded tiny cases
of ``tests.inputs.tiny_case``; nothing here touches the GPU library.  Run from
the repository root:  python -m tests.golden.make_golden
"""

import json
import os

import numpy as np

from oracle import dbf_oracle as O
from tests import inputs

CASES = [
    # seed, n, m, k, batch
    (100, 3, 4, 2, 2),
    (101, 4, 3, 5, 1),
    (102, 6, 5, 4, 3),
    (103, 2, 6, 6, 2),
]


def main():
    out = []
    for seed, n, m, k, batch in CASES:
        X, A, B, a, mid, b = inputs.tiny_case(seed, n, m, k, batch)
        exact = O.brute_force(X, A, B, a, mid, b)
        y64 = np.array([[float(f) for f in row] for row in exact])
        out.append({
            "seed": seed, "n": n, "m": m, "k": k, "batch": batch,
            "y_exact": [[str(f) for f in row] for row in exact],
            "y_fp16_bits": O.rne_fp16(y64).view(np.uint16).tolist(),
        })
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "brute_force_cases.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
