"""fp64 numpy statement of the chunked backward of the KDA recurrence -- the
algebra the device backward kernels evaluate.

Test infrastructure only (like chunk_form.py): nothing on the device path
imports it.  Its agreement with the oracle's token-loop gradient pins the
chunk-level formulas below.

Forward per chunk (one head, C tokens, start state S; e = exp(g),
Gam_r = prod_{u<=r} e_u, gam = Gam_C, D_rs = Gam_r / Gam_s (s <= r), as
products of e over (s, r]):
  M[r,s]  = sum_i k_ri k_si D_rsi (s < r),   A = diag(beta) M
  Pm[r,s] = sum_i q_ri k_si D_rsi (s <= r),  P = scale Pm
  T = (I + A)^-1,  Kd = K*Gam,  Qd = scale Q*Gam,  Ki = K*gam/Gam
  W = T diag(beta) Kd,  U = T diag(beta) V
  Delta = U - W S,  O = Qd S + P Delta,  S' = diag(gam) S + Ki^T Delta
Backward, given dO and dS' (the gradient at the chunk's end):
  dDelta = P^T dO + Ki dS'                       (sequential, with dS)
  dS     = diag(gam) dS' + Qd^T dO - W^T dDelta  (gradient at the start)
  dQd = dO S^T,  dP = tril(dO Delta^T),  dKi = Delta dS'^T,
  dgam = rowsum(dS' * S),  dW = -dDelta S^T,  dU = dDelta
  dT = dU (diag(beta) V)^T + dW (diag(beta) Kd)^T
  dv = beta * (T^T dU),  dKd = beta * (T^T dW)
  dbeta = rowsum(V * T^T dU) + rowsum(Kd * T^T dW) + rowsum(dA * M)
  dA = -T^T dT T^T (strictly lower),  dM = diag(beta) dA,  dPm = scale dP
  through the decayed products (row role r, column role s):
    dk_r += sum_s dM_rs k_s D_rs,   dk_s += sum_r dM_rs k_r D_rs
    dq_r += sum_s dPm_rs k_s D_rs,  dk_s += sum_r dPm_rs q_r D_rs
    dG_r += k_r * (sum_s dM_rs k_s D_rs) + q_r * (sum_s dPm_rs k_s D_rs)
    dG_s -= k_s * (sum_r (dM_rs k_r + dPm_rs q_r) D_rs)
  elementwise:  dk += dKd*Gam + dKi*gam/Gam,  dq += scale dQd*Gam,
    dG += dKd*Kd + dQd*Qd - dKi*Ki,  dG_last += sum_r dKi*Ki + dgam*gam
  and dg_u = sum_{r >= u} dG_r (G_r = sum_{u<=r} g_u).
"""
from __future__ import annotations

import numpy as np


def _decay(e):
    """D[r, s, i] = prod_{u=s+1..r} e_u[i] for s <= r, else 0."""
    C, Dk = e.shape
    D = np.zeros((C, C, Dk))
    for s in range(C):
        p = np.ones(Dk)
        D[s, s] = p
        for r in range(s + 1, C):
            p = p * e[r]
            D[r, s] = p
    return D


def _chunk_fwd(q, k, v, g, beta, S, scale):
    C, Dk = k.shape
    e = np.exp(g)
    D = _decay(e)
    Gam = np.cumprod(e, axis=0)
    gam = Gam[-1]
    suf = np.array([D[C - 1, r] for r in range(C)])  # gam / Gam_r
    M = np.tril(np.einsum("ri,si,rsi->rs", k, k, D), -1)
    Pm = np.tril(np.einsum("ri,si,rsi->rs", q, k, D))
    A = beta[:, None] * M
    T = np.linalg.inv(np.eye(C) + A)
    Kd, Qd, Ki = k * Gam, scale * q * Gam, k * suf
    W = T @ (beta[:, None] * Kd)
    U = T @ (beta[:, None] * v)
    Delta = U - W @ S
    O = Qd @ S + scale * Pm @ Delta
    S_next = gam[:, None] * S + Ki.T @ Delta
    return dict(e=e, D=D, Gam=Gam, gam=gam, suf=suf, M=M, Pm=Pm, A=A, T=T,
                Kd=Kd, Qd=Qd, Ki=Ki, W=W, U=U, Delta=Delta, O=O,
                S_next=S_next)


def _chunk_bwd(q, k, v, g, beta, S, scale, f, dO, dSn):
    """Gradients of one chunk given its forward record f, dO and the
    gradient dSn at the chunk's end.  Returns dq, dk, dv, dg, dbeta, dS."""
    C, Dk = k.shape
    T, D = f["T"], f["D"]
    P = scale * f["Pm"]
    dDelta = P.T @ dO + f["Ki"] @ dSn
    dS = f["gam"][:, None] * dSn + f["Qd"].T @ dO - f["W"].T @ dDelta
    dQd = dO @ S.T
    dP = np.tril(dO @ f["Delta"].T)
    dKi = f["Delta"] @ dSn.T
    dgam = np.sum(dSn * S, axis=1)
    dU, dW = dDelta, -dDelta @ S.T
    BV, BK = beta[:, None] * v, beta[:, None] * f["Kd"]
    dT = dU @ BV.T + dW @ BK.T
    dBV, dBK = T.T @ dU, T.T @ dW
    dv = beta[:, None] * dBV
    dKd = beta[:, None] * dBK
    dA = np.tril(-T.T @ dT @ T.T, -1)
    dbeta = (np.sum(v * dBV, 1) + np.sum(f["Kd"] * dBK, 1)
             + np.sum(dA * f["M"], 1))
    dM = beta[:, None] * dA
    dPm = scale * dP
    # decayed products, row role (r) and column role (s)
    rowK = np.einsum("rs,si,rsi->ri", dM, k, D)
    rowQ = np.einsum("rs,si,rsi->ri", dPm, k, D)
    colK = np.einsum("rs,ri,rsi->si", dM, k, D)
    colQ = np.einsum("rs,ri,rsi->si", dPm, q, D)
    dk = rowK + colK + colQ + dKd * f["Gam"] + dKi * f["suf"]
    dq = rowQ + scale * dQd * f["Gam"]
    dG = (k * rowK + q * rowQ - k * (colK + colQ)
          + dKd * f["Kd"] + dQd * f["Qd"] - dKi * f["Ki"])
    dG[-1] += np.sum(dKi * f["Ki"], 0) + dgam * f["gam"]
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dv, dg, dbeta, dS


def chunked_backward(q, k, v, g, beta, s0, scale, do, dsT=None, C=16):
    """Chunked gradient for [B,T,H,*] inputs (fp64).  Returns
    (dq, dk, dv, dg, dbeta, ds0) like the oracle's backward."""
    B, Tn, H, Dk = q.shape
    Dv = v.shape[-1]
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v),
           np.zeros_like(g), np.zeros_like(beta),
           np.zeros((B, H, Dk, Dv))]
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if s0 is None else s0[b, h].copy()
            recs = []
            for c0 in range(0, Tn, C):
                sl = slice(c0, min(Tn, c0 + C))
                f = _chunk_fwd(q[b, sl, h], k[b, sl, h], v[b, sl, h],
                               g[b, sl, h], beta[b, sl, h], S, scale)
                recs.append((sl, S, f))
                S = f["S_next"]
            dS = np.zeros((Dk, Dv)) if dsT is None else dsT[b, h].copy()
            for sl, S0c, f in reversed(recs):
                r = _chunk_bwd(q[b, sl, h], k[b, sl, h], v[b, sl, h],
                               g[b, sl, h], beta[b, sl, h], S0c, scale, f,
                               do[b, sl, h], dS)
                for o, x in zip(out[:4], r[:4]):
                    o[b, sl, h] = x
                out[4][b, sl, h] = r[4]
                dS = r[5]
            out[5][b, h] = dS
    return tuple(out)
