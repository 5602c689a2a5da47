"""fp64 numpy statement of the chunked (WY / UT-transform) form of the KDA
recurrence -- the algebra the device kernels evaluate in tiles.

It lives in tests/ only: the device path does not import it, and the oracle
is the token loop, not this.  Agreement of this form with the oracle to
~1e-12 pins the chunk algebra (and cross-checks the oracle with a different
evaluation order).

Per head, for a chunk of C tokens r = 1..C starting from state S0
(e_r = exp(g_r) per key channel, Gam_r = prod_{u<=r} e_u):
  A[r,s] = beta_r sum_i k_ri k_si Gam_ri/Gam_si     (s < r)
  P[r,s] = scale sum_i q_ri k_si Gam_ri/Gam_si      (s <= r)
  T      = (I + A)^-1
  W = T diag(beta) (K * Gam),  U = T diag(beta) V
  Delta  = U - W S0                    (beta-scaled corrections)
  O      = scale (Q * Gam) S0 + P Delta
  S_C    = diag(Gam_C) S0 + (K * Gam_C/Gam)^T Delta
The decay ratios are never formed as Gam_r / Gam_s: inside a chunk they are
products of e over (s, r], split at sub-chunk boundaries of `bs` tokens so
each factor is a product of values <= 1 (no overflow, exact for g = -inf).
Diagonal sub-blocks use the sub-chunk start as reference (rho_r / rho_s) when
that ratio is safe, and a direct running product otherwise.
"""
from __future__ import annotations

import numpy as np

SAFE_MIN = 2.0 ** -64


def _decay_between(e, s, r):
    """prod_{u=s+1..r} e_u (vector over key channels), r >= s."""
    return np.prod(e[s + 1:r + 1], axis=0) if r > s else np.ones(e.shape[1])


def chunk_matrices(q, k, g, beta, scale, bs=16):
    """S-independent per-chunk quantities for one head.
    q,k,g: [C, Dk]; beta: [C].  Returns A, P (C x C) and Gam (C x Dk),
    gamC (Dk), Ktil (C x Dk)."""
    C, Dk = k.shape
    e = np.exp(g)
    nb = (C + bs - 1) // bs
    rho = np.ones((C, Dk))   # inclusive prefix within the sub-chunk
    sig = np.ones((C, Dk))   # exclusive suffix within the sub-chunk
    Fs = np.ones((nb, Dk))
    for a in range(nb):
        lo, hi = a * bs, min(C, (a + 1) * bs)
        p = np.ones(Dk)
        for r in range(lo, hi):
            p = p * e[r]
            rho[r] = p
        Fs[a] = p
        p = np.ones(Dk)
        for r in range(hi - 1, lo - 1, -1):
            sig[r] = p
            p = p * e[r]
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for a in range(nb):
        ra = slice(a * bs, min(C, (a + 1) * bs))
        for b in range(a):
            sb = slice(b * bs, min(C, (b + 1) * bs))
            mid = np.prod(Fs[b + 1:a], axis=0) if a - b >= 2 else np.ones(Dk)
            col = k[sb] * sig[sb] * mid        # <= |k|
            A[ra, sb] = (beta[ra, None] * k[ra] * rho[ra]) @ col.T
            P[ra, sb] = scale * (q[ra] * rho[ra]) @ col.T
        # diagonal block
        idx = range(ra.start, ra.stop)
        rr = rho[ra]
        # every rho of the sub-chunk, the last one too: it divides the last
        # token's own column (P's diagonal), so a vanished rho there must
        # take the direct path as well
        if np.all(rr >= SAFE_MIN):
            col = k[ra] / rr
            Ad = (beta[ra, None] * k[ra] * rr) @ col.T
            Pd = scale * (q[ra] * rr) @ col.T
        else:  # direct running products
            n = ra.stop - ra.start
            Ad = np.zeros((n, n))
            Pd = np.zeros((n, n))
            for i, r in enumerate(idx):
                for j, s in enumerate(idx):
                    if s <= r:
                        d = _decay_between(e, s, r)
                        Ad[i, j] = beta[r] * np.sum(k[r] * k[s] * d)
                        Pd[i, j] = scale * np.sum(q[r] * k[s] * d)
        n = ra.stop - ra.start
        A[ra, ra] = np.tril(Ad, -1)
        P[ra, ra] = np.tril(Pd, 0)
        del n
    Fpre = np.ones((nb, Dk))
    Fsuf = np.ones((nb, Dk))
    for a in range(1, nb):
        Fpre[a] = Fpre[a - 1] * Fs[a - 1]
    for a in range(nb - 2, -1, -1):
        Fsuf[a] = Fsuf[a + 1] * Fs[a + 1]
    Gam = np.empty((C, Dk))
    Ktil = np.empty((C, Dk))
    for a in range(nb):
        ra = slice(a * bs, min(C, (a + 1) * bs))
        Gam[ra] = rho[ra] * Fpre[a]
        Ktil[ra] = k[ra] * sig[ra] * Fsuf[a]
    gamC = Fpre[-1] * Fs[-1]
    return A, P, Gam, gamC, Ktil


def chunked_forward(q, k, v, g, beta, s0=None, scale=1.0, C=64, bs=16):
    """Same signature/layout as the oracle's recurrence (fp64 numpy)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    sT = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if s0 is None else s0[b, h].copy()
            for t0 in range(0, T, C):
                sl = slice(t0, min(T, t0 + C))
                qc, kc, vc = q[b, sl, h], k[b, sl, h], v[b, sl, h]
                gc, bc = g[b, sl, h], beta[b, sl, h]
                A, P, Gam, gamC, Kt = chunk_matrices(qc, kc, gc, bc, scale,
                                                     min(bs, C))
                Tm = np.linalg.inv(np.eye(len(bc)) + A)
                W = Tm @ (bc[:, None] * kc * Gam)
                U = Tm @ (bc[:, None] * vc)
                D = U - W @ S
                o[b, sl, h] = scale * (qc * Gam) @ S + P @ D
                S = gamC[:, None] * S + Kt.T @ D
            sT[b, h] = S
    return o, sT


def chunked_forward_scalar_gate(q, k, v, g, beta, s0=None, scale=1.0, C=64):
    """The chunked form with one log-decay per token-head (g [B,T,H]), in
    the arrangement of the per-head-gate chunk prep: Gram products of the
    raw keys and queries times a scalar decay matrix, T applied with its
    columns scaled, and rows of Q and K scaled for the state products.
      D[r,s] = prod_{u=s+1..r} e_u    (s <= r; a direct product, no ratio)
      A = diag(beta) (K K^T * D) (strictly lower), P = scale (Q K^T * D)
      W = T diag(beta Gam) K,  U = T diag(beta) V,  T = (I + A)^-1
      Qtil = scale diag(Gam) Q,  Ktil = diag(Gam_C / Gam) K"""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    sT = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if s0 is None else s0[b, h].copy()
            for t0 in range(0, T, C):
                sl = slice(t0, min(T, t0 + C))
                qc, kc, vc = q[b, sl, h], k[b, sl, h], v[b, sl, h]
                e, bc = np.exp(g[b, sl, h]), beta[b, sl, h]
                n = len(e)
                D = np.zeros((n, n))
                for r in range(n):
                    for s in range(r + 1):
                        D[r, s] = np.prod(e[s + 1:r + 1])
                gam = np.array([np.prod(e[:r + 1]) for r in range(n)])
                sfx = np.array([np.prod(e[r + 1:]) for r in range(n)])
                A = np.tril(bc[:, None] * (kc @ kc.T) * D, -1)
                P = scale * (qc @ kc.T) * D
                Tm = np.linalg.inv(np.eye(n) + A)
                W = (Tm * (bc * gam)[None, :]) @ kc
                U = (Tm * bc[None, :]) @ vc
                Dl = U - W @ S
                o[b, sl, h] = (scale * gam[:, None] * qc) @ S + P @ Dl
                S = gam[-1] * S + (sfx[:, None] * kc).T @ Dl
            sT[b, h] = S
    return o, sT
