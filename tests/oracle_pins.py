"""Pins for the fp64 oracle: checks against what the pages and the
mathematics fix, independent of the oracle's own loop.

Each pin is a function ``pin_x(orc)`` that raises AssertionError on a
mismatch, so the same suite runs against the real oracle
(test_oracle_pins.py) and against deliberately broken copies of it
(test_oracle_mutants.py), where at least one pin must fail.

What each pin fixes (pages: see the header of oracle/kda_oracle.h):
  one_token       S0 = 0, T = 1: o = scale * beta (q.k) v, S = beta k v^T --
                  read-after-update, beta placement, scale placement.
  frozen          beta = 0, g = 0: the state never changes.
  pure_decay      beta = 0: o_t = scale S0^T (exp(G_t) * q_t) with G_t the
                  running sum of g -- per-ROW (key-channel) decay, natural exp.
  forget_restart  g = -inf at t0 on every channel: everything before t0 is
                  forgotten (no NaN); all g = -inf: o_t = beta_t (q_t.k_t) v_t.
  retrieval       |k| = 1, q = k, beta = 1: o_t = v_t -- the delta rule
                  writes exactly the correction ("write only the difference").
  dense_unrolled  S_t = Phi(t,0) S0 + sum_s Phi(t,s) beta_s k_s v_s^T with
                  Phi a product of (I - beta k k^T) diag(exp g) matrices,
                  computed with dense numpy matrix products (brute force).
  contraction     beta in (0,1), |k| = 1, g <= 0: ||S_t|| <= ||S_t-1|| +
                  beta_t ||v_t|| ("the state update is contractive").
  scalar_gate     g equal across channels reduces to the ungated delta rule
                  on values rescaled by the cumulative decay (Gated DeltaNet
                  special case), given as [B,T,H,Dk] and as the per-head
                  [B,T,H] gate.
  neg_eigen       beta in (1,2) ("negative eigenvalues" allowed), g = 0,
                  v = 0, |k| = 1: the k-component of the state is scaled by
                  1 - beta < 0 and the rest is untouched; beta = 2 is a
                  reflection, so the same token twice restores S0.
  linearity       (S0, V) -> (o, S_T) is linear for fixed q, k, g, beta.
  column_split    value columns are independent of each other.
  head_perm       heads and batch rows are independent.
  conv_torch      the conv equals torch.nn.functional.conv1d (groups = C,
                  left padding W-1), with and without a history.
  conv_identity   taps (0,..,0,1) give the identity; the history update.
  l2_numpy        L2 norm equals x / sqrt(||x||^2 + eps) via numpy.linalg.
  conv_prologue   the prologue composition (Oracle.conv_prologue and
                  Oracle.prefill(conv=...)): each stream [B,T,H*D] through
                  torch conv1d, split into heads as [B,T,H,D] (head h owns
                  channels h*D .. h*D+D-1), q and k scaled per head to
                  x / sqrt(||x||^2 + eps) with numpy, v left raw; d_k != d_v,
                  H = 3, with and without a history, per-channel and per-head
                  gates through the prefill.
  bwd_fd          the gradient (backward) equals central finite differences
                  of the forward oracle's loss sum(o*dO) + sum(S_T*dS_T) for
                  every input (q, k, v, g, beta, S0), per-channel and per-head
                  gates, over more than one 64-token checkpoint block.
  bwd_one_token   S0 = 0, T = 1: the closed-form gradient of
                  o = scale beta (q.k) v.
"""
from __future__ import annotations

import numpy as np
import torch

RTOL = 1e-12


def _rand(rng, B, T, H, Dk, Dv, unit_k=True, g_scale=1.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -g_scale * np.log1p(np.exp(rng.standard_normal((B, T, H, Dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.3 * rng.standard_normal((B, H, Dk, Dv))
    return q, k, v, g, beta, s0


def _close(a, b, tol=RTOL, what=""):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)), f"{what}: non-finite"
    den = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / den
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


def pin_one_token(orc):
    rng = np.random.default_rng(1)
    q, k, v, g, beta, _ = _rand(rng, 2, 1, 3, 5, 4, unit_k=False)
    scale = 0.37
    o, s = orc.recurrence(q, k, v, g, beta, None, scale)
    qk = np.einsum("bthi,bthi->bth", q, k)
    _close(o, scale * (beta * qk)[..., None] * v, what="o")
    exp_s = np.einsum("bhi,bhj->bhij", beta[:, 0, :, None] * k[:, 0], v[:, 0])
    _close(s, exp_s, what="S")


def pin_frozen(orc):
    rng = np.random.default_rng(2)
    q, k, v, _, _, s0 = _rand(rng, 2, 7, 2, 6, 3)
    g = np.zeros_like(q)
    beta = np.zeros(q.shape[:3])
    o, s = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    _close(s, s0, what="S")
    _close(o, np.einsum("bhij,bthi->bthj", s0, q), what="o")


def pin_pure_decay(orc):
    rng = np.random.default_rng(3)
    q, k, v, g, _, s0 = _rand(rng, 1, 9, 2, 6, 3)
    beta = np.zeros(q.shape[:3])
    scale = 1.7
    o, s = orc.recurrence(q, k, v, g, beta, s0, scale)
    G = np.cumsum(g, axis=1)  # running log-decay per key channel
    exp_o = scale * np.einsum("bhij,bthi->bthj", s0, np.exp(G) * q)
    _close(o, exp_o, what="o")
    _close(s, np.exp(G[:, -1])[..., None] * s0, what="S")


def pin_forget_restart(orc):
    rng = np.random.default_rng(4)
    q, k, v, g, beta, s0 = _rand(rng, 1, 12, 2, 5, 4)
    t0 = 5
    g[:, t0] = -np.inf
    o, s = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    g2 = g[:, t0:].copy()
    g2[:, 0] = 0.0
    o2, s2 = orc.recurrence(q[:, t0:], k[:, t0:], v[:, t0:], g2,
                            beta[:, t0:], None, 1.0)
    _close(o[:, t0:], o2, what="o after forget")
    _close(s, s2, what="S after forget")
    g[:] = -np.inf
    o, _ = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    qk = np.einsum("bthi,bthi->bth", q, k)
    _close(o, (beta * qk)[..., None] * v, what="o all forgotten")


def pin_retrieval(orc):
    rng = np.random.default_rng(5)
    _, k, v, g, _, s0 = _rand(rng, 2, 10, 2, 8, 5)
    beta = np.ones(k.shape[:3])
    o, _ = orc.recurrence(k, k, v, g, beta, s0, 1.0)
    _close(o, v, tol=1e-11, what="retrieval")


def dense_unrolled(q, k, v, g, beta, s0, scale):
    """Brute force: S_t = Phi(t,0) S0 + sum_{s<=t} Phi(t,s) beta_s k_s v_s^T,
    Phi(t,s) = M_t M_{t-1} ... M_{s+1}, M_r = (I - beta_r k_r k_r^T) diag(e_r),
    Phi(t,t) = I; built from explicit dense matrices (one head at a time)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    sT = np.zeros((B, H, Dk, Dv))
    I = np.eye(Dk)
    for b in range(B):
        for h in range(H):
            M = [(I - beta[b, r, h] * np.outer(k[b, r, h], k[b, r, h]))
                 @ np.diag(np.exp(g[b, r, h])) for r in range(T)]
            for t in range(T):
                Phi = I.copy()  # Phi(t, t)
                St = np.zeros((Dk, Dv))
                for s in range(t, -1, -1):  # s = t, t-1, ..., 0
                    St += Phi @ (beta[b, s, h] * np.outer(k[b, s, h],
                                                          v[b, s, h]))
                    Phi = Phi @ M[s]  # now Phi(t, s-1)
                St += Phi @ s0[b, h]
                o[b, t, h] = scale * St.T @ q[b, t, h]
                if t == T - 1:
                    sT[b, h] = St
    return o, sT


def pin_dense_unrolled(orc):
    rng = np.random.default_rng(6)
    for (T, Dk, Dv) in ((6, 3, 4), (8, 4, 2), (1, 4, 4)):
        q, k, v, g, beta, s0 = _rand(rng, 2, T, 2, Dk, Dv, unit_k=False,
                                     g_scale=0.5)
        o, s = orc.recurrence(q, k, v, g, beta, s0, 0.8)
        eo, es = dense_unrolled(q, k, v, g, beta, s0, 0.8)
        _close(o, eo, tol=1e-11, what=f"o T{T}")
        _close(s, es, tol=1e-11, what=f"S T{T}")


def pin_contraction(orc):
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0 = _rand(rng, 1, 20, 1, 6, 6, g_scale=0.05)
    prev = np.linalg.norm(s0[0, 0], 2)
    s = s0
    for t in range(20):
        sl = slice(t, t + 1)
        _, s = orc.recurrence(q[:, sl], k[:, sl], v[:, sl], g[:, sl],
                              beta[:, sl], s, 1.0)
        cur = np.linalg.norm(s[0, 0], 2)
        bound = prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert cur <= bound * (1 + 1e-12), (t, cur, bound)
        prev = cur


def pin_scalar_gate(orc):
    """Channel-uniform gate a_t: S_t = A_t * Sg_t where Sg runs the ungated
    (g = 0) delta rule on values v_t / A_t, A_t = prod_{u<=t} exp(a_u)."""
    rng = np.random.default_rng(8)
    q, k, v, _, beta, s0 = _rand(rng, 1, 10, 2, 5, 3)
    a = -0.3 * np.abs(rng.standard_normal((1, 10, 2)))
    g = np.repeat(a[..., None], 5, axis=-1)
    o, s = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    A = np.exp(np.cumsum(a, axis=1))
    og, sg = orc.recurrence(q, k, v / A[..., None], np.zeros_like(g), beta,
                            s0, 1.0)
    _close(o, og * A[..., None], tol=1e-11, what="o")
    _close(s, sg * A[:, -1, :, None, None], tol=1e-11, what="S")
    oh, sh = orc.recurrence(q, k, v, a, beta, s0, 1.0)  # per-head layout
    _close(oh, og * A[..., None], tol=1e-11, what="o (per-head gate)")
    _close(sh, sg * A[:, -1, :, None, None], tol=1e-11,
           what="S (per-head gate)")


def pin_neg_eigen(orc):
    """Transition I - beta k k^T with beta in (1,2): eigenvalue 1 - beta on
    k, 1 elsewhere."""
    rng = np.random.default_rng(12)
    Dk, Dv = 6, 4
    k = rng.standard_normal(Dk)
    k /= np.linalg.norm(k)
    s0 = rng.standard_normal((1, 1, Dk, Dv))
    z = np.zeros((1, 1, 1, Dk))
    kk = k.reshape(1, 1, 1, Dk)
    for b in (1.3, 1.9):
        _, s = orc.recurrence(z, kk, np.zeros((1, 1, 1, Dv)), z,
                              np.full((1, 1, 1), b), s0, 1.0)
        _close(k @ s[0, 0], (1.0 - b) * (k @ s0[0, 0]), tol=1e-13,
               what=f"k-component, beta={b}")
        perp = np.eye(Dk) - np.outer(k, k)
        _close(perp @ s[0, 0], perp @ s0[0, 0], tol=1e-13,
               what=f"orthogonal part, beta={b}")
    two = np.full((1, 2, 1), 2.0)
    _, s = orc.recurrence(np.zeros((1, 2, 1, Dk)), np.repeat(kk, 2, axis=1),
                          np.zeros((1, 2, 1, Dv)), np.zeros((1, 2, 1, Dk)),
                          two, s0, 1.0)
    _close(s, s0, tol=1e-13, what="reflection twice")


def pin_linearity(orc):
    rng = np.random.default_rng(9)
    q, k, v, g, beta, s0 = _rand(rng, 1, 8, 2, 4, 3)
    v2 = rng.standard_normal(v.shape)
    s02 = rng.standard_normal(s0.shape)
    o1, s1 = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    o2, s2 = orc.recurrence(q, k, v2, g, beta, s02, 1.0)
    o3, s3 = orc.recurrence(q, k, 2.0 * v - 3.0 * v2, g, beta,
                            2.0 * s0 - 3.0 * s02, 1.0)
    _close(o3, 2.0 * o1 - 3.0 * o2, tol=1e-11, what="o")
    _close(s3, 2.0 * s1 - 3.0 * s2, tol=1e-11, what="S")


def pin_column_split(orc):
    rng = np.random.default_rng(10)
    q, k, v, g, beta, s0 = _rand(rng, 1, 8, 2, 4, 6)
    o, s = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    perm = rng.permutation(6)
    o2, s2 = orc.recurrence(q, k, v[..., perm], g, beta, s0[..., perm], 1.0)
    _close(o2, o[..., perm], what="o")
    _close(s2, s[..., perm], what="S")
    oa, _ = orc.recurrence(q, k, v[..., :2], g, beta, s0[..., :2], 1.0)
    _close(oa, o[..., :2], what="o split")


def pin_head_perm(orc):
    rng = np.random.default_rng(11)
    q, k, v, g, beta, s0 = _rand(rng, 2, 6, 3, 4, 3)
    o, s = orc.recurrence(q, k, v, g, beta, s0, 1.0)
    p = [2, 0, 1]
    o2, s2 = orc.recurrence(q[:, :, p], k[:, :, p], v[:, :, p], g[:, :, p],
                            beta[:, :, p], s0[:, p], 1.0)
    _close(o2, o[:, :, p], what="o heads")
    _close(s2, s[:, p], what="S heads")
    o3, _ = orc.recurrence(q[::-1], k[::-1], v[::-1], g[::-1], beta[::-1],
                           s0[::-1], 1.0)
    _close(o3, o[::-1], what="o batch")


def pin_conv_torch(orc):
    rng = np.random.default_rng(12)
    B, T, C, W = 2, 11, 5, 4
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, W))
    y, _ = orc.causal_conv(x, w)
    xt = torch.from_numpy(x).permute(0, 2, 1)
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :],
                                     groups=C, padding=W - 1)[..., :T]
    _close(y, ref.permute(0, 2, 1).numpy(), what="conv")
    hist = rng.standard_normal((B, C, W - 1))
    y, hout = orc.causal_conv(x, w, hist)
    xcat = torch.cat([torch.from_numpy(hist), xt], dim=-1)
    ref = torch.nn.functional.conv1d(xcat, torch.from_numpy(w)[:, None, :],
                                     groups=C)
    _close(y, ref.permute(0, 2, 1).numpy(), what="conv hist")
    _close(hout, xcat[..., -(W - 1):].numpy(), what="hist out")


def pin_conv_identity(orc):
    rng = np.random.default_rng(13)
    B, T, C, W = 1, 2, 3, 4
    x = rng.standard_normal((B, T, C))
    w = np.zeros((C, W))
    w[:, -1] = 1.0
    hist = rng.standard_normal((B, C, W - 1))
    y, hout = orc.causal_conv(x, w, hist)
    _close(y, x, what="identity")
    # T = 2 < W-1 = 3: the new history keeps the newest old entry
    exp_h = np.concatenate([hist[..., -1:], x.transpose(0, 2, 1)], axis=-1)
    _close(hout, exp_h, what="short-T history")
    w2 = np.zeros((C, W))
    w2[:, 0] = 1.0  # oldest tap: a shift by W-1 steps into the history
    y2, _ = orc.causal_conv(x, w2, hist)
    _close(y2, hist[..., :T].transpose(0, 2, 1), what="shift")


def pin_l2_numpy(orc):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((3, 4, 2, 8))
    eps = 1e-6
    y = orc.l2norm(x, eps)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    _close(y, x / np.sqrt(n * n + eps), what="l2")


def _conv_ref(x, w, hist=None):
    """torch conv1d over [B,T,C] (groups = C, taps newest last), with the
    history prepended or W-1 zeros of left padding."""
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64)).permute(0, 2, 1)
    wt = torch.from_numpy(np.asarray(w, dtype=np.float64))[:, None, :]
    C, W = w.shape
    if hist is None:
        y = torch.nn.functional.conv1d(xt, wt, groups=C,
                                       padding=W - 1)[..., :xt.shape[-1]]
    else:
        xt = torch.cat([torch.from_numpy(hist), xt], dim=-1)
        y = torch.nn.functional.conv1d(xt, wt, groups=C)
    return y.permute(0, 2, 1).numpy()


def pin_conv_prologue(orc):
    rng = np.random.default_rng(15)
    B, T, H, Dk, Dv, W, eps = 2, 9, 3, 4, 6, 4, 1e-6
    xq = rng.standard_normal((B, T, H * Dk))
    xk = rng.standard_normal((B, T, H * Dk))
    xv = rng.standard_normal((B, T, H * Dv))
    # taps differ per channel so a wrong channel-to-head split shows
    wq = 0.5 * rng.standard_normal((H * Dk, W))
    wk = 0.5 * rng.standard_normal((H * Dk, W))
    wv = 0.5 * rng.standard_normal((H * Dv, W))

    def heads_l2(y, D, norm):
        y = y.reshape(B, T, H, D)  # head h = channels [h*D, (h+1)*D)
        if norm:
            n = np.linalg.norm(y, axis=-1, keepdims=True)
            y = y / np.sqrt(n * n + eps)
        return y

    for hist in (None, tuple(rng.standard_normal((B, H * D, W - 1))
                             for D in (Dk, Dk, Dv))):
        hq, hk, hv = (None, None, None) if hist is None else hist
        want = (heads_l2(_conv_ref(xq, wq, hq), Dk, True),
                heads_l2(_conv_ref(xk, wk, hk), Dk, True),
                heads_l2(_conv_ref(xv, wv, hv), Dv, False))
        got = orc.conv_prologue(xq, xk, xv, wq, wk, wv, H, Dk, Dv, eps,
                                True, hist)
        for name, a, b in zip("qkv", got[:3], want):
            _close(a, b, what=f"prologue {name} hist={hist is not None}")
        # without the norm all three streams are the raw conv
        got = orc.conv_prologue(xq, xk, xv, wq, wk, wv, H, Dk, Dv, eps,
                                False, hist)
        _close(got[0], heads_l2(_conv_ref(xq, wq, hq), Dk, False),
               what="prologue q, no norm")
        if hist is not None:
            for i, (x, hh) in enumerate(((xq, hq), (xk, hk), (xv, hv))):
                cat = np.concatenate([hh, x.transpose(0, 2, 1)], axis=-1)
                _close(got[3][i], cat[..., -(W - 1):], what=f"history {i}")
    # the whole forward with the prologue: the recurrence (pinned above) on
    # the q, k, v built here, for a per-channel and a per-head gate
    q, k, v = (heads_l2(_conv_ref(xq, wq), Dk, True),
               heads_l2(_conv_ref(xk, wk), Dk, True),
               heads_l2(_conv_ref(xv, wv), Dv, False))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H, Dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    conv = dict(xq=xq, xk=xk, xv=xv, wq=wq, wk=wk, wv=wv, eps=eps,
                l2norm_qk=True)
    for gate in (g, g[..., 1].copy()):
        o, s = orc.prefill(None, None, None, gate, beta, None, 0.9, conv=conv)
        ro, rs = orc.recurrence(q, k, v, gate, beta, None, 0.9)
        _close(o, ro, what=f"prefill conv o (gate ndim {gate.ndim})")
        _close(s, rs, what=f"prefill conv S (gate ndim {gate.ndim})")


def _fd_check(orc, args, scale, do, dsT, elems, tol, what):
    """Central differences (h = 1e-6) of the forward loss for the chosen
    elements of each argument against orc.backward."""
    names = ("q", "k", "v", "g", "beta", "s0")
    grads = orc.backward(*args, scale, do, dsT)
    order = (0, 1, 2, 3, 4, 5)  # backward returns dq, dk, dv, dg, dbeta, ds0

    def loss(a):
        o, s = orc.recurrence(*a, scale)
        return float((o * do).sum() + (s * dsT).sum())
    h = 1e-6
    for ai, gi in zip(range(6), order):
        gr = grads[gi]
        assert gr.shape == args[ai].shape, (names[ai], gr.shape)
        for ix in elems(args[ai].shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[ai][ix] += h
            am[ai][ix] -= h
            fd = (loss(ap) - loss(am)) / (2 * h)
            den = max(np.max(np.abs(gr)), 1e-12)
            assert abs(fd - gr[ix]) <= tol * den, \
                (what, names[ai], ix, fd, gr[ix])


def pin_bwd_fd(orc):
    rng = np.random.default_rng(21)
    every = lambda shape: list(np.ndindex(shape))
    # tiny: every element, per-channel gate
    q, k, v, g, beta, s0 = _rand(rng, 1, 5, 2, 3, 2)
    do = rng.standard_normal(v.shape)
    dsT = rng.standard_normal(s0.shape)
    _fd_check(orc, [q, k, v, g, beta, s0], 0.7, do, dsT, every, 1e-7,
              "tiny")
    # per-head gate [B,T,H]
    a = g[..., 0].copy()
    _fd_check(orc, [q, k, v, a, beta, s0], 0.7, do, dsT, every, 1e-7,
              "per-head gate")
    # beta in (1,2) and a zero start state
    _fd_check(orc, [q, k, v, g, 1.0 + beta, np.zeros_like(s0)], 1.0, do,
              dsT, every, 1e-7, "beta > 1")
    # across checkpoint blocks: 150 tokens, sampled elements
    q, k, v, g, beta, s0 = _rand(rng, 1, 150, 1, 2, 2, g_scale=0.05)
    do = rng.standard_normal(v.shape)
    dsT = rng.standard_normal(s0.shape)
    pick = np.random.default_rng(5)

    def some(shape):
        flat = pick.choice(int(np.prod(shape)), size=min(12, int(np.prod(shape))),
                           replace=False)
        return [np.unravel_index(f, shape) for f in flat] + \
            [tuple(d - 1 for d in shape), tuple(0 for _ in shape)]
    _fd_check(orc, [q, k, v, g, beta, s0], 1.0, do, dsT, some, 1e-6,
              "150 tokens")


def pin_bwd_one_token(orc):
    rng = np.random.default_rng(22)
    q, k, v, g, beta, _ = _rand(rng, 1, 1, 1, 4, 3)
    do = rng.standard_normal(v.shape)
    sc = 0.6
    dq, dk, dv, dg, db, ds0 = orc.backward(q, k, v, g, beta, None, sc, do)
    b = beta[0, 0, 0]
    qv, kv, vv, dov = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], do[0, 0, 0]
    vd, qk = vv @ dov, qv @ kv
    _close(dq[0, 0, 0], sc * b * vd * kv, tol=1e-14, what="dq")
    _close(dk[0, 0, 0], sc * b * vd * qv, tol=1e-14, what="dk")
    _close(dv[0, 0, 0], sc * b * qk * dov, tol=1e-14, what="dv")
    _close(db[0, 0, 0], sc * qk * vd, tol=1e-14, what="dbeta")
    assert np.all(dg == 0.0), "dg with S0 = 0"
    e = np.exp(g[0, 0, 0])
    want = e[:, None] * (sc * np.outer(qv, dov) - sc * b * qk *
                         np.outer(kv, dov))
    _close(ds0[0, 0], want, tol=1e-14, what="dS0")


ALL_PINS = [pin_one_token, pin_frozen, pin_pure_decay, pin_forget_restart,
            pin_retrieval, pin_dense_unrolled, pin_contraction,
            pin_scalar_gate, pin_neg_eigen, pin_linearity, pin_column_split, pin_head_perm,
            pin_conv_torch, pin_conv_identity, pin_l2_numpy,
            pin_conv_prologue, pin_bwd_fd,
            pin_bwd_one_token]
