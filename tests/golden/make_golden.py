"""Write tests/golden/oracle_tiny.json: a small regression fixture whose
expected values come from the fp64 oracle only (this script calls nothing
but oracle/ and numpy).  The pages print no worked numeric example for the
KDA recurrence, so this fixture is a regression guard for the oracle, not an
independent pin; the pins are in tests/oracle_pins.py.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(20261203)
    B, T, H, Dk, Dv = 1, 6, 2, 3, 2
    q = rng.standard_normal((B, T, H, Dk)).round(3)
    k = rng.standard_normal((B, T, H, Dk)).round(3)
    v = rng.standard_normal((B, T, H, Dv)).round(3)
    g = -np.abs(rng.standard_normal((B, T, H, Dk))).round(3)
    beta = rng.uniform(0.05, 0.95, (B, T, H)).round(3)
    s0 = rng.standard_normal((B, H, Dk, Dv)).round(3)
    o, s = oracle.get().recurrence(q, k, v, g, beta, s0, 0.5)
    out = dict(note="oracle regression fixture (expected values from oracle/ "
                    "only); the pages print no worked example",
               scale=0.5, q=q.tolist(), k=k.tolist(), v=v.tolist(),
               g=g.tolist(), beta=beta.tolist(), s0=s0.tolist(),
               o=o.tolist(), s=s.tolist())
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
