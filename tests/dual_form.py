"""Dual-form TTT in float64 numpy: an independent formulation used to pin the
primal oracle (test helper, not collected by pytest).

Follows "论文速览 | TTT" (equinox-blog), §3.6 (dual form for f = Wx:
W_b = W0 - 2 eta (W0 X - X) X^T, Delta = (W0 X - X) mask(X^T X),
Z = W0 X - 2 eta Delta, with X split into the K / V / Q views of §3.3) and
§3.7 (dual form for MLPs: gradients of the whole mini-batch at the starting
weights, outputs through a causal mask(A^T Q) per layer), with the scalar eta
generalised to the per-token eta_t of §4.6 (column t of the gradient matrix
is scaled by eta_t).  Matrices have tokens as columns (d x b), as on the page.
The causal mask keeps s <= t (the inclusive diagonal: token t's output sees
its own update, §3.1).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def gelu_grad(x):
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def linear_unit(q, k, v, eta, w0, b):
    """One unit: q, k, v [T, d], eta [T], w0 [d, d] -> (z [T, d], W_T)."""
    T, d = q.shape
    W = np.array(w0, dtype=np.float64)
    Z = np.zeros((T, d))
    for m0 in range(0, T, b):
        m1 = min(T, m0 + b)
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        G = 2.0 * (W @ XK - XV) * e[None, :]  # eta_t * dl_t/d(W x) per column
        mask = np.triu(XK.T @ XQ)  # (s, t) kept for s <= t
        Z[m0:m1] = (W @ XQ - G @ mask).T
        W = W - G @ XK.T
    return Z, W


def _ln_columns(Y, eps):
    """Per-column LayerNorm statistics (columns are tokens): normalised Y and
    1 / sqrt(var + eps), population variance."""
    mu = Y.mean(axis=0)
    var = ((Y - mu) ** 2).mean(axis=0)
    rs = 1.0 / np.sqrt(var + eps)
    return (Y - mu) * rs, rs


def linear_ln_unit(q, k, v, eta, w0, gamma, beta, eps, b):
    """One unit of TTT-Linear with the §4.4 LayerNorm + residual wrapper,
    f(x) = x + gamma * LNhat(W x) + beta, in the dual form: the gradients of
    a whole mini-batch at its starting W (the LayerNorm VJP column by column),
    the outputs from W0 Q - G triu(K^T Q) before the output LayerNorm."""
    T, d = q.shape
    W = np.array(w0, dtype=np.float64)
    Z = np.zeros((T, d))
    gc, bc = gamma[:, None], beta[:, None]
    for m0 in range(0, T, b):
        m1 = min(T, m0 + b)
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        Yh, rs = _ln_columns(W @ XK, eps)
        Gh = 2.0 * gc * (XK + gc * Yh + bc - XV)
        GY = rs[None, :] * (Gh - Gh.mean(axis=0) - Yh * (Gh * Yh).mean(axis=0))
        G = GY * e[None, :]
        Oh, _ = _ln_columns(W @ XQ - G @ np.triu(XK.T @ XQ), eps)
        Z[m0:m1] = (XQ + gc * Oh + bc).T
        W = W - G @ XK.T
    return Z, W


def mlp_unit(q, k, v, eta, w1, w2, b):
    """One unit of TTT-MLP, f(x) = W2 GELU(W1 x)."""
    T, d = q.shape
    W1 = np.array(w1, dtype=np.float64)
    W2 = np.array(w2, dtype=np.float64)
    Z = np.zeros((T, d))
    for m0 in range(0, T, b):
        m1 = min(T, m0 + b)
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        # batch forward / backward at the starting weights (App. A)
        Z1 = W1 @ XK
        X2 = gelu(Z1)
        Z2 = W2 @ X2
        G2 = 2.0 * (Z2 - XV) * e[None, :]
        G1 = (W2.T @ G2) * gelu_grad(Z1)
        # outputs: each layer's input matrix A masked against its query side
        Z1q = W1 @ XQ - G1 @ np.triu(XK.T @ XQ)
        X2q = gelu(Z1q)
        Z[m0:m1] = (W2 @ X2q - G2 @ np.triu(X2.T @ X2q)).T
        W1 = W1 - G1 @ XK.T
        W2 = W2 - G2 @ X2.T
    return Z, W1, W2


def mlp_ln_unit(q, k, v, eta, w1, w2, gamma, beta, eps, b):
    """One unit of TTT-MLP with the §4.4 LayerNorm + residual wrapper,
    f(x) = x + gamma * LNhat(W2 GELU(W1 x)) + beta, in the §3.7 dual form:
    the whole mini-batch's gradients at its starting weights, with the
    LayerNorm VJP (column by column) between the loss and the second layer;
    the outputs from the two masked products, then the output LayerNorm."""
    T, d = q.shape
    W1 = np.array(w1, dtype=np.float64)
    W2 = np.array(w2, dtype=np.float64)
    Z = np.zeros((T, d))
    gc, bc = gamma[:, None], beta[:, None]
    for m0 in range(0, T, b):
        m1 = min(T, m0 + b)
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        Z1 = W1 @ XK
        X2 = gelu(Z1)
        Yh, rs = _ln_columns(W2 @ X2, eps)
        Gh = 2.0 * gc * (XK + gc * Yh + bc - XV)
        G2 = rs[None, :] * (Gh - Gh.mean(axis=0) - Yh * (Gh * Yh).mean(axis=0)) * e[None, :]
        G1 = (W2.T @ G2) * gelu_grad(Z1)
        X2q = gelu(W1 @ XQ - G1 @ np.triu(XK.T @ XQ))
        Oh, _ = _ln_columns(W2 @ X2q - G2 @ np.triu(X2.T @ X2q), eps)
        Z[m0:m1] = (XQ + gc * Oh + bc).T
        W1 = W1 - G1 @ XK.T
        W2 = W2 - G2 @ X2.T
    return Z, W1, W2


def mlp_ln(q, k, v, eta, w1, w2, gamma, beta, eps, b):
    B, H, T, d = q.shape
    hd = w1.shape[-2]
    Z = np.zeros((B, H, T, d))
    W1T = np.zeros((B, H, hd, d))
    W2T = np.zeros((B, H, d, hd))
    for bi in range(B):
        for h in range(H):
            a = w1[bi, h] if w1.ndim == 4 else w1[h]
            c = w2[bi, h] if w2.ndim == 4 else w2[h]
            Z[bi, h], W1T[bi, h], W2T[bi, h] = mlp_ln_unit(q[bi, h], k[bi, h], v[bi, h],
                                                          eta[bi, h], a, c, gamma[h], beta[h],
                                                          eps, b)
    return Z, W1T, W2T


def _units(a, lead):
    return a.reshape(lead, *a.shape[2:])


def linear(q, k, v, eta, w0, b):
    B, H, T, d = q.shape
    Z = np.zeros((B, H, T, d))
    WT = np.zeros((B, H, d, d))
    for bi in range(B):
        for h in range(H):
            w = w0[bi, h] if w0.ndim == 4 else w0[h]
            Z[bi, h], WT[bi, h] = linear_unit(q[bi, h], k[bi, h], v[bi, h], eta[bi, h], w, b)
    return Z, WT


def mlp(q, k, v, eta, w1, w2, b):
    B, H, T, d = q.shape
    hd = w1.shape[-2]
    Z = np.zeros((B, H, T, d))
    W1T = np.zeros((B, H, hd, d))
    W2T = np.zeros((B, H, d, hd))
    for bi in range(B):
        for h in range(H):
            a = w1[bi, h] if w1.ndim == 4 else w1[h]
            c = w2[bi, h] if w2.ndim == 4 else w2[h]
            Z[bi, h], W1T[bi, h], W2T[bi, h] = mlp_unit(q[bi, h], k[bi, h], v[bi, h], eta[bi, h],
                                                       a, c, b)
    return Z, W1T, W2T


def linear_ln(q, k, v, eta, w0, gamma, beta, eps, b):
    B, H, T, d = q.shape
    Z = np.zeros((B, H, T, d))
    WT = np.zeros((B, H, d, d))
    for bi in range(B):
        for h in range(H):
            w = w0[bi, h] if w0.ndim == 4 else w0[h]
            Z[bi, h], WT[bi, h] = linear_ln_unit(q[bi, h], k[bi, h], v[bi, h], eta[bi, h], w,
                                                 gamma[h], beta[h], eps, b)
    return Z, WT


def linear_bwd_unit(q, k, v, eta, w0, b, dz, dwT):
    """Adjoint of the dual-form recurrence, one unit, mini-batch by
    mini-batch in reverse.  Per mini-batch (columns are tokens, D = diag eta):
      E = W K - V, G = 2 E D, A = triu(K^T Q), Z = W Q - G A, W' = W - G K^T.
    Given Zb (adjoint of Z) and Wb' (adjoint of W'):
      Gb = -Zb A^T - Wb' K, Eb = 2 Gb D, Ab = triu(-G^T Zb),
      Wb = Wb' + Zb Q^T + Eb K^T, Qb = W^T Zb + K Ab,
      Kb = W^T Eb + Q Ab^T - Wb'^T G, Vb = -Eb, etab_t = sum_i Gb[i,t] 2 E[i,t].
    Returns (dq, dk, dv, deta, dw0)."""
    T, d = q.shape
    Ws = [np.array(w0, dtype=np.float64)]
    blocks = list(range(0, T, b))
    for m0 in blocks:
        m1 = min(T, m0 + b)
        XK, XV = k[m0:m1].T, v[m0:m1].T
        G = 2.0 * (Ws[-1] @ XK - XV) * eta[m0:m1][None, :]
        Ws.append(Ws[-1] - G @ XK.T)
    dq, dk, dv = (np.zeros((T, d)) for _ in range(3))
    deta = np.zeros(T)
    Wb = np.zeros((d, d)) if dwT is None else np.array(dwT, dtype=np.float64)
    for jb in reversed(range(len(blocks))):
        m0 = blocks[jb]
        m1 = min(T, m0 + b)
        W = Ws[jb]
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        E = W @ XK - XV
        G = 2.0 * E * e[None, :]
        A = np.triu(XK.T @ XQ)
        Zb = dz[m0:m1].T
        Gb = -Zb @ A.T - Wb @ XK
        Eb = 2.0 * Gb * e[None, :]
        Ab = np.triu(-G.T @ Zb)
        dq[m0:m1] = (W.T @ Zb + XK @ Ab).T
        dk[m0:m1] = (W.T @ Eb + XQ @ Ab.T - Wb.T @ G).T
        dv[m0:m1] = (-Eb).T
        deta[m0:m1] = np.sum(Gb * 2.0 * E, axis=0)
        Wb = Wb + Zb @ XQ.T + Eb @ XK.T
    return dq, dk, dv, deta, Wb


def gelu_grad2(x):
    return np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi) * (2.0 - x * x)


def mlp_bwd_unit(q, k, v, eta, w1, w2, b, dz, dw1T=None, dw2T=None):
    """Adjoint of the TTT-MLP dual-form recurrence (mlp_unit), one unit,
    mini-batch by mini-batch in reverse.  Per mini-batch (D = diag eta,
    Phi' = GELU', Phi'' = GELU''):
      Z1 = W1 K, X2 = GELU(Z1), Z2 = W2 X2, G2 = 2 (Z2 - V) D,
      S = W2^T G2, G1 = S * Phi'(Z1), A = triu(K^T Q),
      Z1q = W1 Q - G1 A, X2q = GELU(Z1q), B2 = triu(X2^T X2q),
      Z = W2 X2q - G2 B2, W1' = W1 - G1 K^T, W2' = W2 - G2 X2^T.
    Given Zb and W1b', W2b' it takes every product back in reverse order.
    Returns (dq, dk, dv, deta, dw1_0, dw2_0)."""
    T, d = q.shape
    W1s, W2s = [np.array(w1, dtype=np.float64)], [np.array(w2, dtype=np.float64)]
    blocks = list(range(0, T, b))
    for m0 in blocks:
        m1 = min(T, m0 + b)
        XK, XV = k[m0:m1].T, v[m0:m1].T
        Z1 = W1s[-1] @ XK
        X2 = gelu(Z1)
        G2 = 2.0 * (W2s[-1] @ X2 - XV) * eta[m0:m1][None, :]
        G1 = (W2s[-1].T @ G2) * gelu_grad(Z1)
        W1s.append(W1s[-1] - G1 @ XK.T)
        W2s.append(W2s[-1] - G2 @ X2.T)
    dq, dk, dv = (np.zeros((T, d)) for _ in range(3))
    deta = np.zeros(T)
    W1b = np.zeros_like(W1s[0]) if dw1T is None else np.array(dw1T, dtype=np.float64)
    W2b = np.zeros_like(W2s[0]) if dw2T is None else np.array(dw2T, dtype=np.float64)
    for jb in reversed(range(len(blocks))):
        m0 = blocks[jb]
        m1 = min(T, m0 + b)
        W1, W2 = W1s[jb], W2s[jb]
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1][None, :]
        # forward of the mini-batch
        Z1 = W1 @ XK
        X2, D = gelu(Z1), gelu_grad(Z1)
        E = W2 @ X2 - XV
        G2 = 2.0 * E * e
        S = W2.T @ G2
        G1 = S * D
        A = np.triu(XK.T @ XQ)
        Z1q = W1 @ XQ - G1 @ A
        X2q, Dq = gelu(Z1q), gelu_grad(Z1q)
        B2 = np.triu(X2.T @ X2q)
        # adjoints
        Zb = dz[m0:m1].T
        W1n, W2n = W1b.copy(), W2b.copy()  # the state's adjoint passes through
        W2n += Zb @ X2q.T
        Mb = np.triu(-G2.T @ Zb)
        X2b = X2q @ Mb.T - W2b.T @ G2
        X2qb = W2.T @ Zb + X2 @ Mb
        G2b = -Zb @ B2.T - W2b @ X2
        G1b = -W1b @ XK
        Kb = -W1b.T @ G1
        Z1qb = X2qb * Dq
        W1n += Z1qb @ XQ.T
        Qb = W1.T @ Z1qb
        G1b += -Z1qb @ A.T
        Ab = np.triu(-G1.T @ Z1qb)
        Kb += XQ @ Ab.T
        Qb += XK @ Ab
        Sb = G1b * D
        Z1b = G1b * S * gelu_grad2(Z1)
        W2n += G2 @ Sb.T
        G2b += W2 @ Sb
        Eb = 2.0 * G2b * e
        deta[m0:m1] = np.sum(G2b * 2.0 * E, axis=0)
        W2n += Eb @ X2.T
        X2b += W2.T @ Eb
        Z1b += X2b * D
        W1n += Z1b @ XK.T
        Kb += W1.T @ Z1b
        dq[m0:m1], dk[m0:m1], dv[m0:m1] = Qb.T, Kb.T, -Eb.T
        W1b, W2b = W1n, W2n
    return dq, dk, dv, deta, W1b, W2b


def _ln_hat_adjoint(C, rs, Hb, rsb0=0.0):
    """Adjoint of Yh = C rs, C = Y - mean Y, rs = (mean C^2 + eps)^-1/2 per
    column, given Yh's adjoint Hb (and an extra adjoint rsb0 of rs): Y's."""
    d = C.shape[0]
    rsb = rsb0 + np.sum(C * Hb, axis=0)
    varb = -0.5 * rs ** 3 * rsb
    Cb = rs[None, :] * Hb + (2.0 / d) * C * varb[None, :]
    return Cb - Cb.mean(axis=0)


def linear_ln_bwd_unit(q, k, v, eta, w0, gamma, beta, eps, b, dz, dwT=None):
    """Adjoint of linear_ln_unit, one unit, mini-batch by mini-batch in
    reverse, every product of the dual form taken back (columns are tokens,
    D = diag eta, A = triu(K^T Q)):
      Y = W K, Yh = LNhat(Y), R = K + gamma Yh + beta - V, Gh = 2 gamma R,
      P = Gh - mean Gh - Yh mean(Gh Yh), GY = rs P, G = GY D,
      Zp = W Q - G A, Z = Q + gamma LNhat(Zp) + beta, W' = W - G K^T.
    Returns (dq, dk, dv, deta, dw0, dgamma, dbeta)."""
    T, d = q.shape
    gc, bc = gamma[:, None], beta[:, None]
    Ws = [np.array(w0, dtype=np.float64)]
    blocks = list(range(0, T, b))
    for m0 in blocks:
        m1 = min(T, m0 + b)
        XK, XV = k[m0:m1].T, v[m0:m1].T
        Yh, rs = _ln_columns(Ws[-1] @ XK, eps)
        Gh = 2.0 * gc * (XK + gc * Yh + bc - XV)
        G = rs[None, :] * (Gh - Gh.mean(axis=0) - Yh * (Gh * Yh).mean(axis=0)) * eta[m0:m1][None, :]
        Ws.append(Ws[-1] - G @ XK.T)
    dq, dk, dv = (np.zeros((T, d)) for _ in range(3))
    deta = np.zeros(T)
    dgam, dbet = np.zeros(d), np.zeros(d)
    Wb = np.zeros((d, d)) if dwT is None else np.array(dwT, dtype=np.float64)
    for jb in reversed(range(len(blocks))):
        m0 = blocks[jb]
        m1 = min(T, m0 + b)
        W = Ws[jb]
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1][None, :]
        # forward of the mini-batch
        Y = W @ XK
        C = Y - Y.mean(axis=0)
        Yh, rs = _ln_columns(Y, eps)
        R = XK + gc * Yh + bc - XV
        Gh = 2.0 * gc * R
        gbar, m = Gh.mean(axis=0), (Gh * Yh).mean(axis=0)
        P = Gh - gbar - Yh * m
        GY = rs[None, :] * P
        G = GY * e
        A = np.triu(XK.T @ XQ)
        Zp = W @ XQ - G @ A
        Cq = Zp - Zp.mean(axis=0)
        Zh, rsq = _ln_columns(Zp, eps)
        # the output
        Zb = dz[m0:m1].T
        Qb = Zb.copy()
        dgam += np.sum(Zb * Zh, axis=1)
        dbet += np.sum(Zb, axis=1)
        Zpb = _ln_hat_adjoint(Cq, rsq, gc * Zb)
        Wn = Wb + Zpb @ XQ.T
        Qb += W.T @ Zpb
        Gb = -Zpb @ A.T - Wb @ XK       # W' = W - G K^T passes Wb through
        Ab = np.triu(-G.T @ Zpb)
        Kb = XQ @ Ab.T - Wb.T @ G
        Qb += XK @ Ab
        # G = GY D
        GYb = Gb * e
        deta[m0:m1] = np.sum(Gb * GY, axis=0)
        # GY = rs P, P = Gh - gbar - Yh m
        rsb = np.sum(GYb * P, axis=0)
        Pb = rs[None, :] * GYb
        Ghb = Pb + (-Pb.sum(axis=0) / d)[None, :] + Yh * (-(Pb * Yh).sum(axis=0) / d)[None, :]
        Yhb = -Pb * m[None, :] + Gh * (-(Pb * Yh).sum(axis=0) / d)[None, :]
        # Gh = 2 gamma R, R = K + gamma Yh + beta - V
        Rb = 2.0 * gc * Ghb
        dgam += np.sum(2.0 * R * Ghb + Yh * Rb, axis=1)
        dbet += np.sum(Rb, axis=1)
        Kb += Rb
        Yhb += gc * Rb
        Yb = _ln_hat_adjoint(C, rs, Yhb, rsb)
        Wn += Yb @ XK.T
        Kb += W.T @ Yb
        dq[m0:m1], dk[m0:m1], dv[m0:m1] = Qb.T, Kb.T, -Rb.T
        Wb = Wn
    return dq, dk, dv, deta, Wb, dgam, dbet


def linear_bwd(q, k, v, eta, w0, b, dz, dwT=None):
    B, H, T, d = q.shape
    out = [np.zeros((B, H, T, d)) for _ in range(3)] + [np.zeros((B, H, T)), np.zeros((B, H, d, d))]
    for bi in range(B):
        for h in range(H):
            w = w0[bi, h] if w0.ndim == 4 else w0[h]
            r = linear_bwd_unit(q[bi, h], k[bi, h], v[bi, h], eta[bi, h], w, b, dz[bi, h],
                                None if dwT is None else dwT[bi, h])
            for o, x in zip(out, r):
                o[bi, h] = x
    return tuple(out)


def mlp_unit_torch(q, k, v, eta, w1, w2, b):
    """The MLP dual form of mlp_unit in float64 torch, differentiable: one
    unit, q, k, v [T, d], eta [T], w1 [h, d], w2 [d, h] (torch tensors).
    Per mini-batch (columns are tokens, "论文速览 | TTT" §3.7): Z1 = W1 K,
    X2 = GELU(Z1), Z2 = W2 X2, G2 = 2 (Z2 - V) diag(eta),
    G1 = (W2^T G2) * GELU'(Z1), Z1q = W1 Q - G1 triu(K^T Q), X2q = GELU(Z1q),
    Z = W2 X2q - G2 triu(X2^T X2q), W1 -= G1 K^T, W2 -= G2 X2^T."""
    import torch
    c = 1.0 / np.sqrt(2.0)
    gel = lambda x: 0.5 * x * (1.0 + torch.erf(x * c))
    gel_d = lambda x: 0.5 * (1.0 + torch.erf(x * c)) + x * torch.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)
    T = q.shape[0]
    W1, W2 = w1, w2
    outs = []
    for m0 in range(0, T, b):
        m1 = min(T, m0 + b)
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        Z1 = W1 @ XK
        X2 = gel(Z1)
        G2 = 2.0 * (W2 @ X2 - XV) * e[None, :]
        G1 = (W2.T @ G2) * gel_d(Z1)
        Z1q = W1 @ XQ - G1 @ torch.triu(XK.T @ XQ)
        X2q = gel(Z1q)
        outs.append((W2 @ X2q - G2 @ torch.triu(X2.T @ X2q)).T)
        W1 = W1 - G1 @ XK.T
        W2 = W2 - G2 @ X2.T
    return torch.cat(outs, dim=0), W1, W2


def linear_ln_unit_torch(q, k, v, eta, w0, gamma, beta, eps, b):
    """linear_ln_unit in float64 torch, differentiable (one unit; q, k, v
    [T, d], eta [T], w0 [d, d], gamma, beta [d]).  Per mini-batch at its
    starting W (columns are tokens): Y = W K, the LayerNorm VJP of
    2 gamma (K + gamma LNhat(Y) + beta - V) column by column gives G,
    W_b = W - G diag(eta) K^T, and the outputs are
    Q + gamma LNhat(W Q - G diag(eta) triu(K^T Q)) + beta ("论文速览 | TTT"
    §3.6 with the §4.4 wrapper)."""
    import torch

    def lnhat(Y):
        mu = Y.mean(dim=0, keepdim=True)
        var = ((Y - mu) ** 2).mean(dim=0, keepdim=True)
        rs = 1.0 / torch.sqrt(var + eps)
        return (Y - mu) * rs, rs

    T = q.shape[0]
    W = w0
    g_, b_ = gamma[:, None], beta[:, None]
    outs = []
    for m0 in range(0, T, b):
        m1 = min(T, m0 + b)
        XK, XV, XQ = k[m0:m1].T, v[m0:m1].T, q[m0:m1].T
        e = eta[m0:m1]
        Yh, rs = lnhat(W @ XK)
        g = 2.0 * g_ * (XK + g_ * Yh + b_ - XV)
        G = rs * (g - g.mean(dim=0, keepdim=True) - Yh * (g * Yh).mean(dim=0, keepdim=True))
        Ge = G * e[None, :]
        outs.append((XQ + g_ * lnhat(W @ XQ - Ge @ torch.triu(XK.T @ XQ))[0] + b_).T)
        W = W - Ge @ XK.T
    return torch.cat(outs, dim=0), W
