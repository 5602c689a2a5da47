"""Helpers shared by the GPU parity tests.

Error metric (the reading used throughout): for an output tensor x and its
fp64 oracle value r, err = max|x - r| / max|r|, computed separately for the
outputs o and the final state.  The bar is 2e-2 when q/k/v are bf16 and 1e-4
when everything is fp32."""
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
