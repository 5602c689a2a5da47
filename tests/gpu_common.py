"""Helpers shared by the GPU parity tests.

Error metric (the reading used throughout): for an output tensor x and its
fp64 oracle value r, err = max|x - r| / max|r|, computed separately for the
outputs o and the final state.  The bar is 2e-2 when q/k/v are bf16 and 1e-4
when everything is fp32.  Because a tensor-wide max|r| can hide an error in
a head of small magnitude, the tests also take the same metric over each
(batch, head) slab on its own and hold the worst slab to the same bar."""
import sys

import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else x
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / max(den, 1e-300))


def to_cpu64(t):
    return t.detach().cpu().double().numpy()


def head_slice(x, h):
    """[B,T,H,...] -> [B,T,1,...] for head h (CPU fp64 numpy)."""
    return to_cpu64(x[:, :, h:h + 1])


def gpu_available():
    return torch.cuda.is_available()


def slab_err(x, ref, axes):
    """Worst per-slab error: the metric above taken over each slab (the
    index tuple along `axes`, e.g. (0, 2) for (batch, head) of [B,T,H,D],
    (0, 1) for [B,H,Dk,Dv]) with that slab's own max|r|.  Returns
    (worst error, slab index)."""
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else x
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if not np.all(np.isfinite(x)):
        return float("inf"), None
    axes = tuple(axes)
    rest = tuple(i for i in range(x.ndim) if i not in axes)
    d = np.max(np.abs(x - ref), axis=rest)
    m = np.maximum(np.max(np.abs(ref), axis=rest), 1e-300)
    e = d / m
    i = np.unravel_index(int(np.argmax(e)), e.shape)
    return float(e[i]), tuple(int(v) for v in i)


# (test id, output, tensor-wide error, worst slab error, slab, bar) of every
# check() in this session; conftest.py prints them after the run
RESULTS = []


def check(name, x, ref, tol, axes):
    """Assert the tensor-wide metric and the worst (batch, head) slab are
    within tol; prints both."""
    import os
    e = rel_err(x, ref)
    w, at = slab_err(x, ref, axes)
    say(f"  {name}: err {e:.2e}, worst slab {w:.2e} at {at}")
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    RESULTS.append((test.split("::")[-1], name, e, w, at, tol))
    assert e <= tol, (name, e)
    assert w <= tol, (name, "slab", at, w)
    return e, w
