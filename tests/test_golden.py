"""Regression guard: the oracle still reproduces its stored tiny fixture."""
import json
import os

import numpy as np


def test_oracle_golden(orc):
    p = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    d = json.load(open(p))
    a = {n: np.array(d[n]) for n in ("q", "k", "v", "g", "beta", "s0", "o", "s")}
    o, s = orc.recurrence(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"],
                          d["scale"])
    np.testing.assert_allclose(o, a["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(s, a["s"], rtol=0, atol=1e-13)
