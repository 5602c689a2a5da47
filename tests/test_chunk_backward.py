"""The chunked backward algebra (tests/chunk_backward.py, fp64 numpy) agrees
with the oracle's token-loop gradient: several chunks and a ragged tail,
nonzero start state and end-state gradient, beta up to 2, and gates of -inf
(exact forgetting) -- the formulas the device backward evaluates."""
import numpy as np
import pytest

from chunk_backward import chunked_backward
from oracle_pins import _rand


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("T,C,bmax", [(37, 16, 1.0), (40, 8, 2.0),
                                      (16, 16, 1.0)])
def test_chunked_backward_matches_oracle(orc, T, C, bmax):
    rng = np.random.default_rng(31 + T)
    q, k, v, g, beta, s0 = _rand(rng, 2, T, 2, 5, 3)
    beta = beta * bmax
    do = rng.standard_normal(v.shape)
    dsT = rng.standard_normal(s0.shape)
    ref = orc.backward(q, k, v, g, beta, s0, 0.8, do, dsT)
    got = chunked_backward(q, k, v, g, beta, s0, 0.8, do, dsT, C=C)
    for name, a, r in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), got, ref):
        assert _rel(a, r) < 1e-10, (name, _rel(a, r))


def test_chunked_backward_neg_inf(orc):
    rng = np.random.default_rng(44)
    q, k, v, g, beta, s0 = _rand(rng, 1, 30, 1, 4, 3)
    g[:, 7] = -np.inf
    g[:, 19, :, 2] = -np.inf
    do = rng.standard_normal(v.shape)
    ref = orc.backward(q, k, v, g, beta, s0, 1.0, do)
    got = chunked_backward(q, k, v, g, beta, s0, 1.0, do, C=16)
    for name, a, r in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), got, ref):
        assert np.all(np.isfinite(a)), name
        assert _rel(a, r) < 1e-10, (name, _rel(a, r))
