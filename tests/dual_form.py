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
