"""The chunked WY/UT algebra the device kernels evaluate (tests/chunk_form.py,
fp64 numpy) equals the token-loop oracle, for several chunk and sub-chunk
sizes, ragged tails, a nonzero initial state and gates of -inf."""
import numpy as np
import pytest

from chunk_form import chunked_forward, chunked_forward_scalar_gate
from oracle_pins import _rand


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


@pytest.mark.parametrize("C,bs", [(1, 1), (4, 4), (16, 16), (32, 16),
                                  (64, 16), (64, 8)])
def test_chunk_form_matches_oracle(orc, C, bs):
    rng = np.random.default_rng(100 + C + bs)
    q, k, v, g, beta, s0 = _rand(rng, 1, 75, 2, 8, 6)
    o, s = orc.recurrence(q, k, v, g, beta, s0, 0.7)
    oc, sc = chunked_forward(q, k, v, g, beta, s0, 0.7, C=C, bs=bs)
    assert _rel(oc, o) < 1e-11 and _rel(sc, s) < 1e-11


def test_chunk_form_neg_inf_gates(orc):
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0 = _rand(rng, 1, 70, 1, 8, 4)
    g[:, 5, :, :] = -np.inf          # full forget inside a sub-chunk
    g[:, 33, :, 3] = -np.inf         # one channel forgotten
    g[:, 40:44] = -60.0              # strong forgetting: diag fallback path
    g[:, 47, :, 1] = -np.inf         # last token of a sub-chunk (its own
                                     # column divides by its rho)
    o, s = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    oc, sc = chunked_forward(q, k, v, g, beta, s0, 1.0, C=64, bs=16)
    assert np.all(np.isfinite(oc)) and np.all(np.isfinite(sc))
    assert _rel(oc, o) < 1e-11 and _rel(sc, s) < 1e-11


@pytest.mark.parametrize("C", [1, 16, 64])
def test_scalar_gate_chunk_form_matches_oracle(orc, C):
    """The per-head-gate arrangement (Gram of raw keys times a scalar decay
    matrix, scaled T columns) equals the token loop, -inf gates included."""
    rng = np.random.default_rng(200 + C)
    q, k, v, g, beta, s0 = _rand(rng, 2, 90, 2, 8, 5)
    gh = g[..., 0].copy()
    gh[0, 20] = -np.inf
    gh[1, 63] = -np.inf
    o, s = orc.recurrence(q, k, v, gh, beta, s0, 0.8)
    oc, sc = chunked_forward_scalar_gate(q, k, v, gh, beta, s0, 0.8, C=C)
    assert np.all(np.isfinite(oc)) and np.all(np.isfinite(sc))
    assert _rel(oc, o) < 1e-11 and _rel(sc, s) < 1e-11
