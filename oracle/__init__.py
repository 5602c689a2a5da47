"""fp64 CPU oracle for the KDA layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``gated_delta_rule_74_amd`` and imports nothing from it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, OpenMP over
independent heads); this module only builds it and marshals numpy arrays.
Every input is upcast exactly to float64 before the call, so the oracle sees
the same rounded bf16/fp32 values the device path sees.

Sources, readings and layouts: see the header of ``kda_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

# -ffp-contract=off / -fno-fast-math: keep IEEE semantics (exp(-inf) == 0,
# no silent FMA contraction) so the oracle is a literal reading of the loop.
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-shared", "-fPIC"]


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


class Oracle:
    """ctypes view of one compiled oracle library (the real one by default;
    tests may load a deliberately broken copy to show the pins catch it)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.kda_oracle_recurrence.restype = ctypes.c_int
        lib.kda_oracle_recurrence.argtypes = [_I64] * 5 + [_P] * 6 + [
            ctypes.c_double, _P, _P]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [_I64] * 5 + [_P] * 6 + [
            ctypes.c_double] + [_P] * 8
        lib.kda_oracle_causal_conv.restype = None
        lib.kda_oracle_causal_conv.argtypes = [_I64] * 4 + [_P] * 5
        lib.kda_oracle_l2norm.restype = None
        lib.kda_oracle_l2norm.argtypes = [_I64] * 3 + [ctypes.c_double, _P]
        self.lib = lib
        self.last_threads = 1

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _f64(a):
        if a is None:
            return None
        if hasattr(a, "detach"):  # torch tensor -> exact upcast on the CPU
            a = a.detach().cpu().double().numpy()
        return np.ascontiguousarray(a, dtype=np.float64)

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(_P)

    # -- API -------------------------------------------------------------
    def recurrence(self, q, k, v, g, beta, s0=None, scale=1.0):
        """Token loop.  q,k,g [B,T,H,Dk] (g may be [B,T,H]: one log-decay
        per token-head for every row); v [B,T,H,Dv]; beta [B,T,H];
        s0 [B,H,Dk,Dv] or None.  Returns (o [B,T,H,Dv], S_T [B,H,Dk,Dv])."""
        q, k, v, g, beta, s0 = (self._f64(x) for x in (q, k, v, g, beta, s0))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        if g.ndim == 3:
            # one log-decay per token-head (the Gated DeltaNet gate): the
            # same coefficient on every row of the state
            g = np.ascontiguousarray(np.repeat(g[..., None], Dk, axis=-1))
        assert k.shape == q.shape and g.shape == q.shape
        assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H)
        if s0 is not None:
            assert s0.shape == (B, H, Dk, Dv)
        o = np.empty((B, T, H, Dv), np.float64)
        s_out = np.empty((B, H, Dk, Dv), np.float64)
        self.last_threads = self.lib.kda_oracle_recurrence(
            B, T, H, Dk, Dv, self._ptr(q), self._ptr(k), self._ptr(v),
            self._ptr(g), self._ptr(beta), self._ptr(s0), float(scale),
            self._ptr(o), self._ptr(s_out))
        return o, s_out

    def backward(self, q, k, v, g, beta, s0, scale, do, dsT=None):
        """Gradient of the token loop for the loss sum(o*do) + sum(S_T*dsT).
        Shapes as recurrence(); do [B,T,H,Dv], dsT [B,H,Dk,Dv] or None.
        Returns (dq, dk, dv, dg, dbeta, ds0); with a per-head gate g
        [B,T,H] the returned dg is [B,T,H] (summed over the rows it
        multiplies)."""
        q, k, v, g, beta, s0, do, dsT = (self._f64(x) for x in
                                         (q, k, v, g, beta, s0, do, dsT))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        head_gate = g.ndim == 3
        if head_gate:
            g = np.ascontiguousarray(np.repeat(g[..., None], Dk, axis=-1))
        assert k.shape == q.shape and g.shape == q.shape
        assert v.shape == (B, T, H, Dv) and beta.shape == (B, T, H)
        assert do.shape == v.shape
        dq, dk, dg = (np.empty_like(q) for _ in range(3))
        dv = np.empty_like(v)
        dbeta = np.empty_like(beta)
        ds0 = np.empty((B, H, Dk, Dv), np.float64)
        self.last_threads = self.lib.kda_oracle_backward(
            B, T, H, Dk, Dv, self._ptr(q), self._ptr(k), self._ptr(v),
            self._ptr(g), self._ptr(beta), self._ptr(s0), float(scale),
            self._ptr(do), self._ptr(dsT), self._ptr(dq), self._ptr(dk),
            self._ptr(dv), self._ptr(dg), self._ptr(dbeta), self._ptr(ds0))
        if head_gate:
            dg = dg.sum(axis=-1)
        return dq, dk, dv, dg, dbeta, ds0

    def decode_step(self, q, k, v, g, beta, state, scale=1.0):
        """One recurrent step for N independent sequences: q,k,g [N,H,Dk],
        v [N,H,Dv], beta [N,H], state [N,H,Dk,Dv] -> (o, new_state)."""
        q, k, v, g, beta = (self._f64(x)[:, None] for x in (q, k, v, g, beta))
        o, s = self.recurrence(q, k, v, g, beta, self._f64(state), scale)
        return o[:, 0], s

    def causal_conv(self, x, w, hist=None):
        """x [B,T,Cn]; w [Cn,W]; hist [B,Cn,W-1] or None.
        Returns (y [B,T,Cn], hist_out [B,Cn,W-1])."""
        x, w, hist = self._f64(x), self._f64(w), self._f64(hist)
        B, T, Cn = x.shape
        W = w.shape[1]
        assert w.shape == (Cn, W)
        y = np.empty_like(x)
        hist_out = np.empty((B, Cn, max(W - 1, 0)), np.float64)
        self.lib.kda_oracle_causal_conv(B, T, Cn, W, self._ptr(x),
                                        self._ptr(w), self._ptr(hist),
                                        self._ptr(y), self._ptr(hist_out))
        return y, hist_out

    def l2norm(self, x, eps):
        """Per-head L2 normalisation of x [..., H, D] (returns a copy)."""
        x = np.array(self._f64(x), dtype=np.float64, copy=True)
        H, D = x.shape[-2:]
        R = int(np.prod(x.shape[:-2]))
        self.lib.kda_oracle_l2norm(R, H, D, float(eps), self._ptr(x))
        return x

    def conv_prologue(self, xq, xk, xv, wq, wk, wv, H, Dk, Dv, eps=1e-6,
                      l2norm_qk=True, hist=None):
        """Conv (+ L2 on q, k) prologue.  x* [B,T,H*D]; w* [H*D, W];
        hist: optional tuple of three [B,H*D,W-1] histories.
        Returns q,k [B,T,H,Dk], v [B,T,H,Dv] and the three new histories."""
        outs, hists = [], []
        for i, (x, w, D) in enumerate(((xq, wq, Dk), (xk, wk, Dk),
                                       (xv, wv, Dv))):
            y, h_out = self.causal_conv(x, w, None if hist is None else hist[i])
            B, T, _ = y.shape
            y = y.reshape(B, T, H, D)
            if l2norm_qk and i < 2:
                y = self.l2norm(y, eps)
            outs.append(y)
            hists.append(h_out)
        return outs[0], outs[1], outs[2], hists

    def prefill(self, q, k, v, g, beta, s0=None, scale=1.0, conv=None):
        """Whole layer forward: optional conv prologue, then the recurrence.
        conv: dict(xq, xk, xv, wq, wk, wv, eps, l2norm_qk) or None."""
        if conv is not None:
            # heads from beta [B,T,H], so g may be per channel [B,T,H,Dk]
            # or per head [B,T,H]; head sizes from the raw channel counts
            H = beta.shape[2]
            Dk = conv["xq"].shape[-1] // H
            Dv = conv["xv"].shape[-1] // H
            q, k, v, _ = self.conv_prologue(
                conv["xq"], conv["xk"], conv["xv"], conv["wq"], conv["wk"],
                conv["wv"], H, Dk, Dv, conv.get("eps", 1e-6),
                conv.get("l2norm_qk", True))
        return self.recurrence(q, k, v, g, beta, s0, scale)


_DEFAULT = None


def get() -> Oracle:
    """The oracle library, compiled on first use if it is not there yet."""
    global _DEFAULT
    if _DEFAULT is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _DEFAULT = Oracle(_LIB)
    return _DEFAULT
