"""Pins for the fp64 primal oracle (CPU only).

The pages print no numeric example of the scan, so the oracle is pinned by
identities the pages and the mathematics fix, each cited to
"论文速览 | TTT" (equinox-blog close reading of "Learning to (Learn at Test
Time): RNNs with Expressive Hidden States"):

* primal == dual form (§3.6 for TTT-Linear, §3.7 / App. A for TTT-MLP);
* Theorem 1 (§4.1): f = Wx, batch GD, eta = 1/2, W0 = 0 is causal linear
  attention z_t = sum_{s<=t} v_s k_s^T q_t;
* b = 1 is online GD, i.e. the delta rule of DeltaNet (§2.6, §3.5);
* b >= T is batch GD, W_t = W0 - eta sum_{s<=t} G_s (§3.5);
* eta = 0 leaves the state at W0 (then Z = W0 Q);
* one mini-batch equals one gradient step on sum_s eta_s l_s, checked against
  central finite differences of the loss (§3.5 / §3.6 closed form);
* Figure 4 (§3.2): one step lowers the current token's loss; for f = Wx the
  ratio is exactly (1 - 2 eta ||k||^2)^2;
* hand-worked scalar examples (tests/golden/scalar_worked_examples.json);
* MLP special cases: zero state stays zero; W2_0 = 0 with b = T is a
  kernelised linear attention with feature map GELU(W1_0 x);
* LayerNorm + residual wrapper (§4.4) of TTT-Linear: primal == a batched dual
  form; one mini-batch equals one gradient step through the LayerNorm
  (central differences); gamma = 0 freezes the state and gives z = q + beta;
  with eps = 0 the scan is covariant under (W0, eta) -> (a W0, a^2 eta)
  (LayerNorm is scale-free, its VJP scales as 1/a); with gamma = 1, beta = 0,
  eps = 0 every output minus its query has mean 0 and variance 1;
* the inner learning-rate gate (§4.6) eta = eta_base sigmoid(theta_lr . x):
  logits placed exactly through one-hot gate vectors give the closed values
  sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4, 1/4, sigmoid(+-ln 7) = 7/8, 1/8 and
  saturation at eta_base, each at its own (batch, head, token); its
  backward (dtheta_lr, dx from deta) against central finite differences of
  sum deta * eta, and the closed form at theta_lr = 0 (sigmoid' = 1/4);
* the LayerNorm scan's backward (§6.12 with §4.4), gamma and beta included:
  central finite differences through the forward oracle, torch's float64
  autodiff of the independently written dual form, and the eta = 0 closed
  forms;
* the TTT-MLP backward (§6.12): central finite differences of
  <dZ, Z> + <dW1_T, W1_T> + <dW2_T, W2_T> through the forward oracle, torch's
  float64 autodiff of the independently written dual form, and the eta = 0
  closed forms (the state never moves);
* invariants: homogeneity, superposition, row permutation, state passing,
  thread-count determinism.

``test_planted_mistakes_are_caught`` rebuilds the oracle with one plausible
mistake at a time (dropped factor 2, wrong sign, output before the update,
gradient at the wrong state, transposed operand, ...) and checks that the pin
set rejects every one of them.

* GELU of the MLP inner model (§4.4 names GELU without a form; read as
  x Phi(x)): GELU(a) and GELU'(a) at a in {0, +-1, +-2}, and GELU''(0), exposed
  one per hidden unit through the MLP's output and both layers' updates, against
  the closed normal-distribution values of
  tests/golden/normal_distribution_values.json (Phi(1), Phi(2), phi(1), phi(2),
  sqrt(2/pi)), which ``test_normal_values_fixture`` re-derives from Taylor series
  in 40-digit decimal arithmetic.  The dual form and the finite-difference check
  share the oracle's definition; this pin does not, so a mistake common to
  GELU and GELU' (erf(x) for erf(x/sqrt 2), the tanh approximation) fails it.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import tempfile

import numpy as np
import pytest

import dual_form
from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_linear(rng, B, H, T, d, eta_scale=0.1, w_scale=0.2, per_batch=False):
    q = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    eta = rng.uniform(0.0, eta_scale, (B, H, T))
    w0 = rng.standard_normal((B, H, d, d) if per_batch else (H, d, d)) * w_scale
    return q, k, v, eta, w0


def rand_mlp(rng, B, H, T, d, hd, eta_scale=0.1, w_scale=0.3):
    q, k, v, eta, _ = rand_linear(rng, B, H, T, d, eta_scale)
    w1 = rng.standard_normal((H, hd, d)) * w_scale
    w2 = rng.standard_normal((H, d, hd)) * w_scale
    return q, k, v, eta, w1, w2


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# Pin functions: each takes an oracle library handle (so the planted-mistake
# test can run them against mutated builds) and raises AssertionError on a
# mismatch.
# ---------------------------------------------------------------------------

def pin_linear_primal_equals_dual(lib):
    rng = np.random.default_rng(11)
    for (T, b) in [(37, 4), (32, 16), (20, 1), (9, 64), (48, 48)]:
        q, k, v, eta, w0 = rand_linear(rng, 2, 2, T, 6)
        z, w = oracle.linear(q, k, v, eta, w0, b, lib=lib)
        zd, wd = dual_form.linear(q, k, v, eta, w0, b)
        assert rel(z, zd) < 1e-12 and rel(w, wd) < 1e-12, (T, b, rel(z, zd), rel(w, wd))


def pin_mlp_primal_equals_dual(lib):
    rng = np.random.default_rng(12)
    for (T, b) in [(23, 4), (16, 16), (7, 1), (10, 32)]:
        q, k, v, eta, w1, w2 = rand_mlp(rng, 1, 2, T, 5, 9, eta_scale=0.5)
        z, a, c = oracle.mlp(q, k, v, eta, w1, w2, b, lib=lib)
        zd, ad, cd = dual_form.mlp(q, k, v, eta, w1, w2, b)
        for x, y in ((z, zd), (a, ad), (c, cd)):
            assert rel(x, y) < 1e-12, (T, b, rel(x, y))


def pin_theorem1_linear_attention(lib):
    rng = np.random.default_rng(13)
    T, d = 24, 5
    q, k, v, _, _ = rand_linear(rng, 1, 1, T, d)
    eta = np.full((1, 1, T), 0.5)
    z, w = oracle.linear(q, k, v, eta, np.zeros((1, d, d)), T, lib=lib)
    # recurrent form of causal linear attention: S_t = S_{t-1} + v_t k_t^T, z_t = S_t q_t
    S = np.zeros((d, d))
    zt = np.zeros((T, d))
    for t in range(T):
        S = S + np.outer(v[0, 0, t], k[0, 0, t])
        zt[t] = S @ q[0, 0, t]
    assert rel(z[0, 0], zt) < 1e-13 and rel(w[0, 0], S) < 1e-13


def pin_b1_delta_rule(lib):
    rng = np.random.default_rng(14)
    T, d = 30, 6
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d, eta_scale=0.5)
    z, w = oracle.linear(q, k, v, eta, w0, 1, lib=lib)
    # DeltaNet's rule: W_t = W_{t-1} (I - beta k k^T) + beta v k^T with beta = 2 eta
    W = w0[0].copy()
    zt = np.zeros((T, d))
    for t in range(T):
        kk, beta = k[0, 0, t], 2.0 * eta[0, 0, t]
        W = W @ (np.eye(d) - beta * np.outer(kk, kk)) + beta * np.outer(v[0, 0, t], kk)
        zt[t] = W @ q[0, 0, t]
    assert rel(z[0, 0], zt) < 1e-12 and rel(w[0, 0], W) < 1e-12


def pin_bT_batch_gd(lib):
    rng = np.random.default_rng(15)
    T, d = 17, 4
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d, eta_scale=0.5)
    for b in (T, 2 * T):
        z, w = oracle.linear(q, k, v, eta, w0, b, lib=lib)
        W0 = w0[0]
        G = np.stack([2.0 * np.outer(W0 @ k[0, 0, t] - v[0, 0, t], k[0, 0, t]) for t in range(T)])
        Wt = W0[None] - np.cumsum(eta[0, 0][:, None, None] * G, axis=0)
        zt = np.einsum("tij,tj->ti", Wt, q[0, 0])
        assert rel(z[0, 0], zt) < 1e-12 and rel(w[0, 0], Wt[-1]) < 1e-12


def pin_eta_zero(lib):
    rng = np.random.default_rng(16)
    q, k, v, eta, w0 = rand_linear(rng, 2, 3, 19, 5)
    eta[:] = 0.0
    z, w = oracle.linear(q, k, v, eta, w0, 4, lib=lib)
    assert np.array_equal(w, np.broadcast_to(w0, w.shape))
    assert rel(z, np.einsum("hij,bhtj->bhti", w0, q)) < 1e-14


def pin_one_step_is_gradient_step(lib):
    """T = b: W_T = W0 - grad_W sum_s eta_s ||W k_s - v_s||^2 at W0 (finite differences)."""
    rng = np.random.default_rng(17)
    T, d = 5, 4
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d, eta_scale=0.5)
    _, w = oracle.linear(q, k, v, eta, w0, T, lib=lib)
    K, V, e, W0 = k[0, 0], v[0, 0], eta[0, 0], w0[0]

    def L(W):
        r = K @ W.T - V
        return float(np.sum(e * np.sum(r * r, axis=1)))

    grad = np.zeros((d, d))
    h = 1e-3
    for i in range(d):
        for j in range(d):
            E = np.zeros((d, d))
            E[i, j] = h
            grad[i, j] = (L(W0 + E) - L(W0 - E)) / (2 * h)
    assert rel(w[0, 0], W0 - grad) < 1e-9


def pin_fig4_loss_ratio(lib):
    rng = np.random.default_rng(18)
    T, d = 12, 5
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d, eta_scale=0.5)
    for t in (1, 5, 11):
        _, w_prev = oracle.linear(q[:, :, :t], k[:, :, :t], v[:, :, :t], eta[:, :, :t], w0, 1, lib=lib)
        _, w_next = oracle.linear(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1],
                                  eta[:, :, :t + 1], w0, 1, lib=lib)
        kk, vv, et = k[0, 0, t], v[0, 0, t], eta[0, 0, t]
        before = np.sum((w_prev[0, 0] @ kk - vv) ** 2)
        after = np.sum((w_next[0, 0] @ kk - vv) ** 2)
        assert abs(after / before - (1.0 - 2.0 * et * kk @ kk) ** 2) < 1e-10


def pin_golden_scalar_examples(lib):
    with open(os.path.join(HERE, "golden", "scalar_worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        T = len(c["eta"])
        sh = lambda key: np.asarray(c[key], dtype=np.float64).reshape(1, 1, T, c["d"])
        z, w = oracle.linear(sh("q"), sh("k"), sh("v"), np.asarray(c["eta"]).reshape(1, 1, T),
                             np.asarray(c["w0"]).reshape(1, c["d"], c["d"]), c["b"], lib=lib)
        assert np.array_equal(z.reshape(T, c["d"]), np.asarray(c["z"])), c["name"]
        assert np.array_equal(w.reshape(c["d"], c["d"]), np.asarray(c["w_T"])), c["name"]


def pin_mlp_one_step_finite_differences(lib):
    rng = np.random.default_rng(19)
    T, d, hd = 4, 3, 5
    q, k, v, eta, w1, w2 = rand_mlp(rng, 1, 1, T, d, hd, eta_scale=0.5, w_scale=0.8)
    _, a, c = oracle.mlp(q, k, v, eta, w1, w2, T, lib=lib)
    K, V, e = k[0, 0], v[0, 0], eta[0, 0]

    def L(W1, W2):
        r = dual_form.gelu(K @ W1.T) @ W2.T - V
        return float(np.sum(e * np.sum(r * r, axis=1)))

    h = 1e-5
    for W, out, which in ((w1[0], a[0, 0], 0), (w2[0], c[0, 0], 1)):
        g = np.zeros_like(W)
        for idx in np.ndindex(*W.shape):
            E = np.zeros_like(W)
            E[idx] = h
            if which == 0:
                g[idx] = (L(W + E, w2[0]) - L(W - E, w2[0])) / (2 * h)
            else:
                g[idx] = (L(w1[0], W + E) - L(w1[0], W - E)) / (2 * h)
        assert rel(out, W - g) < 1e-8, which


def pin_mlp_zero_state(lib):
    rng = np.random.default_rng(20)
    q, k, v, eta, w1, w2 = rand_mlp(rng, 1, 2, 11, 4, 6)
    z, a, c = oracle.mlp(q, k, v, eta, 0 * w1, 0 * w2, 4, lib=lib)
    assert not z.any() and not a.any() and not c.any()


def pin_mlp_w2_zero_kernel_attention(lib):
    rng = np.random.default_rng(21)
    T, d, hd = 9, 4, 6
    q, k, v, eta, w1, w2 = rand_mlp(rng, 1, 1, T, d, hd, eta_scale=0.5)
    z, a, c = oracle.mlp(q, k, v, eta, w1, 0 * w2, T, lib=lib)
    phi = lambda x: dual_form.gelu(w1[0] @ x)
    S = np.zeros((d, hd))
    zt = np.zeros((T, d))
    for t in range(T):
        S = S + 2.0 * eta[0, 0, t] * np.outer(v[0, 0, t], phi(k[0, 0, t]))
        zt[t] = S @ phi(q[0, 0, t])
    assert rel(z[0, 0], zt) < 1e-12 and rel(c[0, 0], S) < 1e-12
    assert np.array_equal(a[0, 0], w1[0])


def _normal_table():
    """Phi, phi at 0, +-1, +-2 and sqrt(2/pi) from tests/golden (closed values)."""
    with open(os.path.join(HERE, "golden", "normal_distribution_values.json")) as f:
        g = json.load(f)
    Phi, phi = {0: 0.5}, {0: float(g["sqrt_2_over_pi"]) / 2.0}
    for s in ("1", "2"):
        a = int(s)
        Phi[a], Phi[-a] = float(g["Phi"][s]), 1.0 - float(g["Phi"][s])
        phi[a] = phi[-a] = float(g["phi"][s])
    return Phi, phi, float(g["sqrt_2_over_pi"])


GELU_POINTS = (0, 1, -1, 2, -2)


def pin_mlp_gelu_closed_values(lib):
    """GELU and GELU' of the oracle's MLP against closed normal-distribution values.

    d = hidden = 5, W2_0 = I; hidden unit u sees the pre-activation
    a_u = W1_0[u][0] k_0 with k = e_0, so every quantity of the MLP is exposed
    per unit:
      * z = W2 GELU(W1 q) with eta = 0, W1 = I, q = points  -> GELU(points);
      * one step (T = b = 1, eta = 1/2), v_u = GELU(a_u) - 1/2 so that the
        output error e = 2 (W2 GELU(a) - v) is 1 in every component:
        W1_T[u][0] = a_u - GELU'(a_u) / 2 and W2_T[i][u] = [i = u] - GELU(a_u) / 2;
      * GELU''(0) = sqrt(2/pi) by a central difference of GELU' at +-h.
    No value of the GELU is computed in this test: the expected values are the
    closed ones of tests/golden/normal_distribution_values.json.
    """
    Phi, phi, s2pi = _normal_table()
    pts = np.array(GELU_POINTS, dtype=np.float64)
    gelu = np.array([a * Phi[a] for a in GELU_POINTS])
    dgelu = np.array([Phi[a] + a * phi[a] for a in GELU_POINTS])
    n = len(pts)
    eye = np.eye(n).reshape(1, n, n)
    zeros = np.zeros((1, 1, 1, n))

    # GELU through the output, eta = 0
    z, _, _ = oracle.mlp(pts.reshape(1, 1, 1, n), zeros, zeros, np.zeros((1, 1, 1)), eye, eye, 1,
                         lib=lib)
    assert np.abs(z[0, 0, 0] - gelu).max() < 1e-15, (z[0, 0, 0], gelu)

    # GELU' through the first layer's update, GELU again through the second's
    w1 = np.zeros((1, n, n))
    w1[0, :, 0] = pts
    k = np.zeros((1, 1, 1, n))
    k[..., 0] = 1.0
    v = (gelu - 0.5).reshape(1, 1, 1, n)
    _, a, c = oracle.mlp(zeros, k, v, np.full((1, 1, 1), 0.5), w1, eye, 1, lib=lib)
    assert np.abs((pts - a[0, 0, :, 0]) * 2.0 - dgelu).max() < 1e-14, (a[0, 0, :, 0], dgelu)
    assert np.abs(a[0, 0, :, 1:]).max() == 0.0
    assert np.abs((np.eye(n) - c[0, 0]) * 2.0 - np.broadcast_to(gelu, (n, n))).max() < 1e-14

    # GELU''(0) = sqrt(2/pi): GELU'(h) - GELU'(-h) over 2h (error ~ (2/3) phi(0) h^2)
    h = 1e-3
    w1 = np.zeros((1, 2, 2))
    w1[0, :, 0] = (h, -h)
    k2 = np.zeros((1, 1, 1, 2))
    k2[..., 0] = 1.0
    eye2 = np.eye(2).reshape(1, 2, 2)
    # v = GELU(+-h) - 1/2 to first order: e = 1 + O(h^2), its effect cancels in the difference
    v2 = np.array([h * 0.5, -h * 0.5]).reshape(1, 1, 1, 2) - 0.5
    _, a2, _ = oracle.mlp(np.zeros((1, 1, 1, 2)), k2, v2, np.full((1, 1, 1), 0.5), w1, eye2, 1,
                          lib=lib)
    dg = (np.array([h, -h]) - a2[0, 0, :, 0]) * 2.0
    assert abs((dg[0] - dg[1]) / (2 * h) - s2pi) < 1e-5 * s2pi, ((dg[0] - dg[1]) / (2 * h), s2pi)


def rand_ln(rng, H, d, g_scale=0.3, b_scale=0.2):
    gamma = 1.0 + g_scale * rng.standard_normal((H, d))
    beta = b_scale * rng.standard_normal((H, d))
    return gamma, beta


def pin_ln_primal_equals_dual(lib):
    rng = np.random.default_rng(31)
    for b in (1, 3, 4, 16):
        q, k, v, eta, w0 = rand_linear(rng, 2, 2, 21, 6, eta_scale=0.3)
        gamma, beta = rand_ln(rng, 2, 6)
        zp, wp = oracle.linear_ln(q, k, v, eta, w0, gamma, beta, 1e-5, b, lib=lib)
        zd, wd = dual_form.linear_ln(q, k, v, eta, w0, gamma, beta, 1e-5, b)
        assert rel(zp, zd) < 1e-12 and rel(wp, wd) < 1e-12, b


def pin_ln_one_step_finite_differences(lib):
    rng = np.random.default_rng(32)
    T, d = 3, 5
    q, k, v, eta, w0 = rand_linear(rng, 1, 1, T, d, eta_scale=0.5, w_scale=0.5)
    gamma, beta = rand_ln(rng, 1, d)
    eps = 1e-3
    _, w1 = oracle.linear_ln(q, k, v, eta, w0, gamma, beta, eps, T, lib=lib)
    K, V, e, g, bb = k[0, 0], v[0, 0], eta[0, 0], gamma[0], beta[0]

    def L(W):
        Y = K @ W.T  # tokens as rows
        mu = Y.mean(axis=1, keepdims=True)
        var = ((Y - mu) ** 2).mean(axis=1, keepdims=True)
        r = K + g * (Y - mu) / np.sqrt(var + eps) + bb - V
        return float(np.sum(e * np.sum(r * r, axis=1)))

    h = 1e-6
    grad = np.zeros((d, d))
    for idx in np.ndindex(d, d):
        E = np.zeros((d, d))
        E[idx] = h
        grad[idx] = (L(w0[0] + E) - L(w0[0] - E)) / (2 * h)
    assert rel(w1[0, 0], w0[0] - grad) < 1e-8


def pin_mlp_ln_primal_equals_dual(lib):
    """TTT-MLP with the LayerNorm + residual wrapper: the primal oracle against
    the dual form of tests/dual_form.py ("论文速览 | TTT" §3.7 with §4.4)."""
    rng = np.random.default_rng(131)
    for b in (1, 3, 4, 16):
        q, k, v, eta, w1, w2 = rand_mlp(rng, 2, 2, 21, 6, 10, eta_scale=0.3)
        gamma, beta = rand_ln(rng, 2, 6)
        zp, ap, cp = oracle.mlp_ln(q, k, v, eta, w1, w2, gamma, beta, 1e-5, b, lib=lib)
        zd, ad, cd = dual_form.mlp_ln(q, k, v, eta, w1, w2, gamma, beta, 1e-5, b)
        assert rel(zp, zd) < 1e-12 and rel(ap, ad) < 1e-12 and rel(cp, cd) < 1e-12, b


def pin_mlp_ln_one_step_finite_differences(lib):
    """One mini-batch (b = T) is one gradient step of sum_s eta_s l_s on both
    layers, l_s = ||k_s + LN(W2 GELU(W1 k_s)) - v_s||^2, checked by central
    differences (Richardson-extrapolated) of that loss written out here."""
    from scipy.special import erf
    rng = np.random.default_rng(132)
    T, d, hd = 3, 4, 5
    q, k, v, eta, w1, w2 = rand_mlp(rng, 1, 1, T, d, hd, eta_scale=0.5, w_scale=0.6)
    gamma, beta = rand_ln(rng, 1, d)
    eps = 1e-3
    _, a1, a2 = oracle.mlp_ln(q, k, v, eta, w1, w2, gamma, beta, eps, T, lib=lib)
    K, V, e, g, bb = k[0, 0], v[0, 0], eta[0, 0], gamma[0], beta[0]

    def L(W1, W2):
        A = K @ W1.T
        Y = (0.5 * A * (1.0 + erf(A / np.sqrt(2.0)))) @ W2.T  # tokens as rows
        mu = Y.mean(axis=1, keepdims=True)
        var = ((Y - mu) ** 2).mean(axis=1, keepdims=True)
        r = K + g * (Y - mu) / np.sqrt(var + eps) + bb - V
        return float(np.sum(e * np.sum(r * r, axis=1)))

    def grad(f, X):
        out = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            def c(h):
                E = np.zeros_like(X)
                E[idx] = h
                return (f(X + E) - f(X - E)) / (2 * h)
            h = 1e-4
            out[idx] = (4.0 * c(h / 2) - c(h)) / 3.0
        return out

    g1 = grad(lambda W: L(W, w2[0]), w1[0])
    g2 = grad(lambda W: L(w1[0], W), w2[0])
    assert rel(a1[0, 0], w1[0] - g1) < 1e-7 and rel(a2[0, 0], w2[0] - g2) < 1e-7


def pin_mlp_ln_gamma_zero(lib):
    """gamma = 0: the LayerNorm passes no gradient, both layers stay put and
    z = q + beta exactly."""
    rng = np.random.default_rng(133)
    q, k, v, eta, w1, w2 = rand_mlp(rng, 2, 2, 13, 6, 8, eta_scale=0.5)
    _, beta = rand_ln(rng, 2, 6)
    z, a, c = oracle.mlp_ln(q, k, v, eta, w1, w2, np.zeros((2, 6)), beta, 1e-5, 4, lib=lib)
    assert np.array_equal(a, np.broadcast_to(w1, a.shape))
    assert np.array_equal(c, np.broadcast_to(w2, c.shape))
    assert np.array_equal(z, q + beta[None, :, None, :])


def pin_mlp_ln_normalised_outputs(lib):
    """gamma = 1, beta = 0, eps = 0: z - q is a normalised vector per token
    (zero mean, unit population variance over the d components)."""
    rng = np.random.default_rng(134)
    q, k, v, eta, w1, w2 = rand_mlp(rng, 2, 2, 17, 6, 8, eta_scale=0.3)
    z, _, _ = oracle.mlp_ln(q, k, v, eta, w1, w2, np.ones((2, 6)), np.zeros((2, 6)), 0.0, 4, lib=lib)
    r = z - q
    assert np.abs(r.mean(axis=-1)).max() < 1e-12
    assert np.abs((r * r).mean(axis=-1) - 1.0).max() < 1e-10


def pin_ln_gamma_zero(lib):
    rng = np.random.default_rng(33)
    q, k, v, eta, w0 = rand_linear(rng, 2, 2, 13, 6, eta_scale=0.5)
    _, beta = rand_ln(rng, 2, 6)
    z, w = oracle.linear_ln(q, k, v, eta, w0, np.zeros((2, 6)), beta, 1e-5, 4, lib=lib)
    assert np.array_equal(w, np.broadcast_to(w0, w.shape))
    assert np.array_equal(z, q + beta[None, :, None, :])


def pin_ln_scale_covariance(lib):
    rng = np.random.default_rng(34)
    q, k, v, eta, w0 = rand_linear(rng, 1, 2, 29, 6, eta_scale=0.2)
    gamma, beta = rand_ln(rng, 2, 6)
    a = 3.0
    z1, w1 = oracle.linear_ln(q, k, v, eta, w0, gamma, beta, 0.0, 4, lib=lib)
    z2, w2 = oracle.linear_ln(q, k, v, a * a * eta, a * w0, gamma, beta, 0.0, 4, lib=lib)
    assert rel(z2, z1) < 1e-12 and rel(w2, a * w1) < 1e-12


def pin_ln_normalised_outputs(lib):
    rng = np.random.default_rng(35)
    q, k, v, eta, w0 = rand_linear(rng, 2, 1, 19, 8, eta_scale=0.3)
    z, _ = oracle.linear_ln(q, k, v, eta, w0, np.ones((1, 8)), np.zeros((1, 8)), 0.0, 4, lib=lib)
    y = z - q
    assert np.abs(y.mean(axis=-1)).max() < 1e-13
    assert np.abs((y * y).mean(axis=-1) - 1.0).max() < 1e-12


# ---- decode steps (§6.11: generation runs the primal form token by token)

def _replay(step_fn, T, B, b, starts):
    """Runs step_fn(t_index, pos) for t = 0..T-1 with each batch element's
    positions starting at its own multiple of b (same mini-batch alignment as
    a scan from token 0)."""
    for t in range(T):
        step_fn(t, np.asarray(starts) + t)


def pin_linear_step_replays_scan(lib):
    rng = np.random.default_rng(41)
    for (T, b) in [(23, 4), (20, 1), (19, 3), (35, 16)]:
        B, H, d = 2, 2, 6
        q, k, v, eta, w0 = rand_linear(rng, B, H, T, d)
        zs, ws = oracle.linear(q, k, v, eta, w0, b, lib=lib)
        w = np.broadcast_to(w0[None], (B, H, d, d)).copy()
        wg = rng.standard_normal(w.shape)  # overwritten at the first step (pos % b == 0)
        z = np.zeros_like(zs)
        st = {"w": w, "wg": wg}

        def step(t, pos):
            zt, st["w"], st["wg"] = oracle.linear_step(q[:, :, t], k[:, :, t], v[:, :, t],
                                                       eta[:, :, t], st["w"], st["wg"], pos, b,
                                                       lib=lib)
            z[:, :, t] = zt
        _replay(step, T, B, b, [0, 2 * b])
        assert rel(z, zs) < 1e-12 and rel(st["w"], ws) < 1e-12, (T, b)


def pin_ln_step_replays_scan(lib):
    rng = np.random.default_rng(42)
    for (T, b) in [(21, 4), (18, 1), (33, 16)]:
        B, H, d = 2, 2, 6
        q, k, v, eta, w0 = rand_linear(rng, B, H, T, d, eta_scale=0.3)
        gamma, beta = rand_ln(rng, H, d)
        zs, ws = oracle.linear_ln(q, k, v, eta, w0, gamma, beta, 1e-5, b, lib=lib)
        st = {"w": np.broadcast_to(w0[None], (B, H, d, d)).copy(),
              "wg": rng.standard_normal((B, H, d, d))}
        z = np.zeros_like(zs)

        def step(t, pos):
            zt, st["w"], st["wg"] = oracle.linear_ln_step(q[:, :, t], k[:, :, t], v[:, :, t],
                                                          eta[:, :, t], st["w"], st["wg"], pos,
                                                          gamma, beta, 1e-5, b, lib=lib)
            z[:, :, t] = zt
        _replay(step, T, B, b, [3 * b, 0])
        assert rel(z, zs) < 1e-12 and rel(st["w"], ws) < 1e-12, (T, b)


def pin_mlp_step_replays_scan(lib):
    rng = np.random.default_rng(43)
    for (T, b) in [(13, 4), (9, 1)]:
        B, H, d, hd = 2, 1, 4, 8
        q, k, v, eta, w1, w2 = rand_mlp(rng, B, H, T, d, hd)
        zs, w1s, w2s = oracle.mlp(q, k, v, eta, w1, w2, b, lib=lib)
        st = {"w1": np.broadcast_to(w1[None], (B, H, hd, d)).copy(),
              "w2": np.broadcast_to(w2[None], (B, H, d, hd)).copy(),
              "w1g": np.zeros((B, H, hd, d)), "w2g": np.zeros((B, H, d, hd))}
        z = np.zeros_like(zs)

        def step(t, pos):
            zt, st["w1"], st["w2"], st["w1g"], st["w2g"] = oracle.mlp_step(
                q[:, :, t], k[:, :, t], v[:, :, t], eta[:, :, t], st["w1"], st["w2"], st["w1g"],
                st["w2g"], pos, b, lib=lib)
            z[:, :, t] = zt
        _replay(step, T, B, b, [b, 0])
        assert rel(z, zs) < 1e-12, (T, b)
        assert rel(st["w1"], w1s) < 1e-12 and rel(st["w2"], w2s) < 1e-12, (T, b)


def pin_step_resumes_a_scan_mid_sequence(lib):
    # A scan over the first m*b tokens ends at the gradient point of the next
    # mini-batch; decode steps continue from there (also mid-mini-batch).
    rng = np.random.default_rng(44)
    B, H, T, d, b, m = 1, 3, 30, 5, 4, 3
    q, k, v, eta, w0 = rand_linear(rng, B, H, T, d)
    zs, ws = oracle.linear(q, k, v, eta, w0, b, lib=lib)
    _, w_mid = oracle.linear(q[:, :, :m * b], k[:, :, :m * b], v[:, :, :m * b],
                             eta[:, :, :m * b], w0, b, lib=lib)
    w, wg = w_mid, np.full_like(w_mid, np.nan)  # a NaN gradient point must never be read
    for t in range(m * b, T):
        zt, w, wg = oracle.linear_step(q[:, :, t], k[:, :, t], v[:, :, t], eta[:, :, t], w, wg,
                                       [t], b, lib=lib)
        assert rel(zt, zs[:, :, t]) < 1e-12, t
    assert rel(w, ws) < 1e-12


def pin_step_golden_scalar_examples(lib):
    with open(os.path.join(HERE, "golden", "scalar_worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        T, d = len(c["eta"]), c["d"]
        w = np.asarray(c["w0"], dtype=np.float64).reshape(1, 1, d, d)
        wg = np.zeros_like(w)
        for t in range(T):
            vec = lambda key: np.asarray(c[key][t], dtype=np.float64).reshape(1, 1, d)
            zt, w, wg = oracle.linear_step(vec("q"), vec("k"), vec("v"),
                                           np.asarray([[c["eta"][t]]]), w, wg, [t], c["b"],
                                           lib=lib)
            assert np.array_equal(zt.reshape(d), np.asarray(c["z"][t])), (c["name"], t)
        assert np.array_equal(w.reshape(d, d), np.asarray(c["w_T"])), c["name"]


# ---- backward of the TTT-Linear scan (§6.12: the outer loop differentiates
# through the inner one)

def _bwd_case(rng, B, H, T, d, per_batch=False):
    q, k, v, eta, w0 = rand_linear(rng, B, H, T, d, eta_scale=0.4, w_scale=0.3,
                                   per_batch=per_batch)
    dz = rng.standard_normal((B, H, T, d))
    dwT = rng.standard_normal((B, H, d, d))
    return q, k, v, eta, w0, dz, dwT


def pin_linear_bwd_finite_differences(lib):
    # L = <dz, Z> + <dwT, W_T>; the backward must give its gradient: compared
    # with central differences of the forward oracle along random directions
    rng = np.random.default_rng(61)
    for (T, b) in [(11, 3), (9, 1), (12, 16), (13, 4)]:
        B, H, d = 1, 2, 4
        q, k, v, eta, w0, dz, dwT = _bwd_case(rng, B, H, T, d)
        grads = oracle.linear_bwd(q, k, v, eta, w0, b, dz, dwT, lib=lib)
        base = dict(q=q, k=k, v=v, eta=eta, w0=w0)

        def L(**kw):
            a = dict(base, **kw)
            z, w = oracle.linear(a["q"], a["k"], a["v"], a["eta"], a["w0"], b, lib=lib)
            return float(np.sum(dz * z) + np.sum(dwT * w))
        h = 1e-5
        for name, g in zip(("q", "k", "v", "eta"), grads[:4]):
            u = rng.standard_normal(base[name].shape)
            fd = (L(**{name: base[name] + h * u}) - L(**{name: base[name] - h * u})) / (2 * h)
            assert abs(fd - np.sum(g * u)) <= 1e-7 * max(1.0, abs(fd)), (name, T, b, fd, np.sum(g * u))
        u = rng.standard_normal(w0.shape)  # shared initial state: the gradient sums over the batch
        fd = (L(w0=w0 + h * u) - L(w0=w0 - h * u)) / (2 * h)
        assert abs(fd - np.sum(grads[4].sum(axis=0) * u)) <= 1e-7 * max(1.0, abs(fd)), ("w0", T, b)


def pin_linear_bwd_equals_dual_form_adjoint(lib):
    rng = np.random.default_rng(62)
    for (T, b, pb) in [(37, 4, False), (32, 16, True), (20, 1, False), (19, 48, False)]:
        q, k, v, eta, w0, dz, dwT = _bwd_case(rng, 2, 2, T, 6, per_batch=pb)
        a = oracle.linear_bwd(q, k, v, eta, w0, b, dz, dwT, lib=lib)
        r = dual_form.linear_bwd(q, k, v, eta, w0, b, dz, dwT)
        for name, x, y in zip(("dq", "dk", "dv", "deta", "dw0"), a, r):
            assert rel(x, y) < 1e-11, (name, T, b, rel(x, y))
        a0 = oracle.linear_bwd(q, k, v, eta, w0, b, dz, None, lib=lib)
        r0 = dual_form.linear_bwd(q, k, v, eta, w0, b, dz, None)
        assert all(rel(x, y) < 1e-11 for x, y in zip(a0, r0)), (T, b)


def pin_linear_bwd_eta_zero(lib):
    # eta = 0: Z = W0 Q, W_T = W0, so dq = W0^T dz, dk = dv = 0 and
    # dw0 = dwT + sum_t dz_t q_t^T; deta_t is the derivative at eta = 0.
    rng = np.random.default_rng(63)
    q, k, v, eta, w0, dz, dwT = _bwd_case(rng, 1, 1, 10, 5)
    eta = np.zeros_like(eta)
    dq, dk, dv, deta, dw0 = oracle.linear_bwd(q, k, v, eta, w0, 4, dz, dwT, lib=lib)
    W = w0[0]
    assert rel(dq[0, 0], dz[0, 0] @ W) < 1e-13
    assert np.abs(dk).max() == 0.0 and np.abs(dv).max() == 0.0
    assert rel(dw0[0, 0], dwT[0, 0] + dz[0, 0].T @ q[0, 0]) < 1e-13


# sigmoid values known in closed form: logit -> sigmoid
_GATE_LOGITS = {0.0: 0.5, np.log(3.0): 0.75, -np.log(3.0): 0.25, np.log(7.0): 0.875,
                -np.log(7.0): 0.125, 60.0: 1.0, -60.0: 0.0}


def _mlp_bwd_case(rng, T, d, hd, with_dwT=True):
    q, k, v, eta, w1, w2 = rand_mlp(rng, 1, 2, T, d, hd, eta_scale=0.5, w_scale=0.5)
    dz = rng.standard_normal(q.shape)
    d1 = rng.standard_normal((1, 2, hd, d)) if with_dwT else None
    d2 = rng.standard_normal((1, 2, d, hd)) if with_dwT else None
    return q, k, v, eta, w1, w2, dz, d1, d2


def pin_mlp_bwd_finite_differences(lib):
    """The MLP backward against central finite differences of
    L = <dZ, Z> + <dW1_T, W1_T> + <dW2_T, W2_T> through the forward oracle,
    along a random direction of every input ("论文速览 | TTT" §6.12)."""
    rng = np.random.default_rng(41)
    for (T, b, with_dwT) in [(7, 3, True), (6, 1, True), (5, 8, False), (9, 9, True)]:
        q, k, v, eta, w1, w2, dz, d1, d2 = _mlp_bwd_case(rng, T, 3, 5, with_dwT)
        g = oracle.mlp_bwd(q, k, v, eta, w1, w2, b, dz, d1, d2, lib=lib)
        base = dict(q=q, k=k, v=v, eta=eta, w1=w1, w2=w2)

        def L(**kw):
            a = dict(base, **kw)
            z, s1, s2 = oracle.mlp(a["q"], a["k"], a["v"], a["eta"], a["w1"], a["w2"], b, lib=lib)
            out = np.sum(dz * z)
            if with_dwT:
                out += np.sum(d1 * s1) + np.sum(d2 * s2)
            return out

        h = 1e-5
        grads = dict(q=g[0], k=g[1], v=g[2], eta=g[3], w1=g[4].sum(axis=0), w2=g[5].sum(axis=0))
        for name, arr in base.items():
            D = rng.standard_normal(arr.shape)
            fd = (L(**{name: arr + h * D}) - L(**{name: arr - h * D})) / (2 * h)
            an = float(np.sum(grads[name] * D))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, T, b, fd, an)


def pin_mlp_bwd_equals_autograd_of_dual_form(lib):
    """The MLP backward equals torch's reverse-mode autodiff (float64) of the
    independently written dual form (tests/dual_form.py, §3.7)."""
    import torch
    rng = np.random.default_rng(42)
    for (T, b) in [(9, 4), (8, 8), (5, 1), (11, 16)]:
        q, k, v, eta, w1, w2, dz, d1, d2 = _mlp_bwd_case(rng, T, 4, 6)
        g = oracle.mlp_bwd(q, k, v, eta, w1, w2, b, dz, d1, d2, lib=lib)
        for h in range(2):
            leaves = [torch.tensor(a, dtype=torch.float64, requires_grad=True)
                      for a in (q[0, h], k[0, h], v[0, h], eta[0, h], w1[h], w2[h])]
            z, s1, s2 = dual_form.mlp_unit_torch(*leaves, b)
            tot = ((z * torch.from_numpy(dz[0, h])).sum() + (s1 * torch.from_numpy(d1[0, h])).sum()
                   + (s2 * torch.from_numpy(d2[0, h])).sum())
            tot.backward()
            for i, leaf in enumerate(leaves):
                assert rel(g[i][0, h], leaf.grad.numpy()) < 1e-11, (T, b, h, i)


def pin_mlp_bwd_equals_dual_form_adjoint(lib):
    """The MLP backward equals the hand-written adjoint of the dual form
    (tests/dual_form.py: every product of one mini-batch taken back in
    reverse, the form a dual-form backward kernel evaluates), float64."""
    rng = np.random.default_rng(44)
    for (T, b) in [(16, 16), (21, 16), (10, 4), (7, 1), (13, 8)]:
        q, k, v, eta, w1, w2, dz, d1, d2 = _mlp_bwd_case(rng, T, 4, 6)
        g = oracle.mlp_bwd(q, k, v, eta, w1, w2, b, dz, d1, d2, lib=lib)
        for h in range(2):
            r = dual_form.mlp_bwd_unit(q[0, h], k[0, h], v[0, h], eta[0, h], w1[h], w2[h], b,
                                       dz[0, h], d1[0, h], d2[0, h])
            for i in range(6):
                assert rel(g[i][0, h], r[i]) < 1e-12, (T, b, h, i)


def pin_mlp_bwd_eta_zero(lib):
    """eta = 0: the state never moves, so z_t = W2_0 GELU(W1_0 q_t) and the
    adjoints are closed forms: dk = dv = 0, dq_t = W1_0^T (GELU'(W1_0 q_t) *
    W2_0^T dz_t), dW2_0 = dW2_T + sum_t dz_t GELU(W1_0 q_t)^T,
    dW1_0 = dW1_T + sum_t (GELU'(W1_0 q_t) * W2_0^T dz_t) q_t^T."""
    rng = np.random.default_rng(43)
    q, k, v, eta, w1, w2, dz, d1, d2 = _mlp_bwd_case(rng, 13, 4, 6)
    eta[:] = 0.0
    g = oracle.mlp_bwd(q, k, v, eta, w1, w2, 4, dz, d1, d2, lib=lib)
    assert not g[1].any() and not g[2].any()
    for h in range(2):
        aq = q[0, h] @ w1[h].T                                   # [T, hd]
        daq = dual_form.gelu_grad(aq) * (dz[0, h] @ w2[h])       # [T, hd]
        assert rel(g[0][0, h], daq @ w1[h]) < 1e-13
        assert rel(g[5][0, h], d2[0, h] + dz[0, h].T @ dual_form.gelu(aq)) < 1e-13
        assert rel(g[4][0, h], d1[0, h] + daq.T @ q[0, h]) < 1e-13


def _ln_bwd_case(rng, T, d, with_dwT=True):
    q, k, v, eta, w0 = rand_linear(rng, 1, 2, T, d, eta_scale=0.3, w_scale=0.5)
    gamma, beta = rand_ln(rng, 2, d)
    dz = rng.standard_normal(q.shape)
    dwT = rng.standard_normal((1, 2, d, d)) if with_dwT else None
    return q, k, v, eta, w0, gamma, beta, dz, dwT


def pin_ln_bwd_finite_differences(lib):
    """The LayerNorm scan's backward against central finite differences of
    L = <dZ, Z> + <dW_T, W_T> through the forward oracle along a random
    direction of every input, gamma and beta included (§6.12, §4.4)."""
    rng = np.random.default_rng(44)
    eps = 1e-3
    for (T, b, with_dwT) in [(7, 3, True), (6, 1, True), (5, 8, False), (9, 9, True)]:
        q, k, v, eta, w0, gamma, beta, dz, dwT = _ln_bwd_case(rng, T, 4, with_dwT)
        g = oracle.linear_ln_bwd(q, k, v, eta, w0, gamma, beta, eps, b, dz, dwT, lib=lib)
        base = dict(q=q, k=k, v=v, eta=eta, w0=w0, gamma=gamma, beta=beta)

        def L(**kw):
            a = dict(base, **kw)
            z, w = oracle.linear_ln(a["q"], a["k"], a["v"], a["eta"], a["w0"], a["gamma"],
                                    a["beta"], eps, b, lib=lib)
            return np.sum(dz * z) + (np.sum(dwT * w) if with_dwT else 0.0)

        h = 1e-4
        grads = dict(q=g[0], k=g[1], v=g[2], eta=g[3], w0=g[4].sum(axis=0),
                     gamma=g[5].sum(axis=0), beta=g[6].sum(axis=0))
        for name, arr in base.items():
            D = rng.standard_normal(arr.shape)
            cd = lambda s: (L(**{name: arr + s * D}) - L(**{name: arr - s * D})) / (2 * s)
            fd = (4.0 * cd(h / 2) - cd(h)) / 3.0  # Richardson: the h^2 term cancels
            an = float(np.sum(grads[name] * D))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, T, b, fd, an)


def pin_ln_bwd_equals_autograd_of_dual_form(lib):
    """The LayerNorm scan's backward equals torch's float64 reverse-mode
    autodiff of the independently written dual form (tests/dual_form.py)."""
    import torch
    rng = np.random.default_rng(45)
    eps = 1e-3
    for (T, b) in [(9, 4), (8, 8), (5, 1), (11, 16)]:
        q, k, v, eta, w0, gamma, beta, dz, dwT = _ln_bwd_case(rng, T, 5)
        g = oracle.linear_ln_bwd(q, k, v, eta, w0, gamma, beta, eps, b, dz, dwT, lib=lib)
        for h in range(2):
            leaves = [torch.tensor(a, dtype=torch.float64, requires_grad=True)
                      for a in (q[0, h], k[0, h], v[0, h], eta[0, h], w0[h], gamma[h], beta[h])]
            z, w = dual_form.linear_ln_unit_torch(*leaves, eps, b)
            ((z * torch.from_numpy(dz[0, h])).sum() + (w * torch.from_numpy(dwT[0, h])).sum()).backward()
            for i, leaf in enumerate(leaves):
                assert rel(g[i][0, h], leaf.grad.numpy()) < 1e-11, (T, b, h, i)


def pin_ln_bwd_equals_dual_form_adjoint(lib):
    """The LayerNorm backward equals the hand-written adjoint of the dual form
    (tests/dual_form.py: every product of one mini-batch taken back in reverse,
    with the LayerNorm VJP's own adjoint), float64."""
    rng = np.random.default_rng(46)
    for (T, b) in [(16, 16), (21, 16), (10, 4), (7, 1), (13, 8)]:
        q, k, v, eta, w0, gamma, beta, dz, dwT = _ln_bwd_case(rng, T, 6)
        g = oracle.linear_ln_bwd(q, k, v, eta, w0, gamma, beta, 1e-3, b, dz, dwT, lib=lib)
        for h in range(2):
            r = dual_form.linear_ln_bwd_unit(q[0, h], k[0, h], v[0, h], eta[0, h], w0[h], gamma[h],
                                             beta[h], 1e-3, b, dz[0, h], dwT[0, h])
            for i in range(7):
                assert rel(g[i][0, h], r[i]) < 1e-12, (T, b, h, i)


def pin_ln_bwd_eta_zero(lib):
    """eta = 0: the state never moves, z_t = q_t + gamma LNhat(W0 q_t) + beta,
    so dk = dv = 0, dbeta = sum_t dz_t, dgamma = sum_t LNhat(W0 q_t) dz_t and
    dq_t = dz_t + W0^T J_t (gamma dz_t), with J_t the LayerNorm Jacobian's
    transpose applied column by column (rs (x - mean x - yh mean(x yh)))."""
    rng = np.random.default_rng(46)
    eps = 1e-3
    q, k, v, eta, w0, gamma, beta, dz, dwT = _ln_bwd_case(rng, 11, 5)
    eta[:] = 0.0
    g = oracle.linear_ln_bwd(q, k, v, eta, w0, gamma, beta, eps, 4, dz, dwT, lib=lib)
    assert not g[1].any() and not g[2].any()
    for h in range(2):
        Y = q[0, h] @ w0[h].T                                         # [T, d]
        mu = Y.mean(axis=1, keepdims=True)
        rs = 1.0 / np.sqrt(((Y - mu) ** 2).mean(axis=1, keepdims=True) + eps)
        Yh = (Y - mu) * rs
        x = gamma[h] * dz[0, h]
        dY = rs * (x - x.mean(axis=1, keepdims=True) - Yh * (x * Yh).mean(axis=1, keepdims=True))
        assert rel(g[0][0, h], dz[0, h] + dY @ w0[h]) < 1e-13
        assert rel(g[6][0, h], dz[0, h].sum(axis=0)) < 1e-13
        assert rel(g[5][0, h], (Yh * dz[0, h]).sum(axis=0)) < 1e-13
        assert rel(g[4][0, h], dwT[0, h] + dY.T @ q[0, h]) < 1e-13


def pin_gate_closed_forms(lib):
    # theta_lr[h] = c_h e_{p(h)} puts the logit c_h x[b, t, p(h)] at every
    # (b, h, t) on its own; each logit is drawn from the closed-form table, so
    # a wrong index, sign or scale shows up as a wrong table value.
    rng = np.random.default_rng(70)
    B, T, H, dx = 2, 5, 3, 8
    keys = list(_GATE_LOGITS)
    pick = rng.integers(0, len(keys), size=(B, H, T))
    perm = [5, 1, 6]  # p(h): the column of x that head h reads
    scale = [1.0, -2.0, 0.5]
    theta = np.zeros((H, dx))
    x = rng.standard_normal((B, T, dx))
    want = np.zeros((B, H, T))
    for h in range(H):
        theta[h, perm[h]] = scale[h]
    for bi in range(B):
        for t in range(T):
            for h in range(H):
                a = keys[pick[bi, h, t]]
                x[bi, t, perm[h]] = a / scale[h]
                want[bi, h, t] = _GATE_LOGITS[a]
    eta_base = 0.37
    got = oracle.lr_gate(x, theta, eta_base, lib=lib)
    assert np.abs(got - eta_base * want).max() < 1e-15
    # a gate vector spread over several inputs: the dot product sums them
    theta2 = np.ones((1, dx)) / dx
    x2 = np.full((1, 1, dx), np.log(3.0))
    assert abs(oracle.lr_gate(x2, theta2, 1.0, lib=lib)[0, 0, 0] - 0.75) < 1e-15
    # theta_lr = 0 gives eta_base / 2 everywhere
    assert np.all(oracle.lr_gate(x, np.zeros((H, dx)), 2.0, lib=lib) == 1.0)


def pin_gate_bwd_finite_differences(lib):
    # L = sum deta * eta(theta, x): the backward must be its gradient
    rng = np.random.default_rng(71)
    B, T, H, dx = 2, 3, 3, 5
    x = rng.standard_normal((B, T, dx))
    theta = rng.standard_normal((H, dx)) * 0.6
    deta = rng.standard_normal((B, H, T))
    eta_base = 0.7
    dth, dxo = oracle.lr_gate_bwd(x, theta, eta_base, deta, lib=lib)
    L = lambda xx, tt: float((deta * oracle.lr_gate(xx, tt, eta_base, lib=lib)).sum())
    h = 1e-6
    fd_t = np.zeros_like(theta)
    for i in np.ndindex(theta.shape):
        e = np.zeros_like(theta)
        e[i] = h
        fd_t[i] = (L(x, theta + e) - L(x, theta - e)) / (2 * h)
    fd_x = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        e = np.zeros_like(x)
        e[i] = h
        fd_x[i] = (L(x + e, theta) - L(x - e, theta)) / (2 * h)
    assert rel(dth, fd_t) < 1e-7 and rel(dxo, fd_x) < 1e-7


def pin_gate_bwd_zero_vector(lib):
    # theta_lr = 0: every logit is 0, sigmoid' = 1/4, so
    # dtheta[h] = eta_base / 4 * sum_{b,t} deta[b,h,t] x[b,t] and dx = 0
    rng = np.random.default_rng(72)
    B, T, H, dx = 2, 4, 3, 6
    x = rng.standard_normal((B, T, dx))
    deta = rng.standard_normal((B, H, T))
    dth, dxo = oracle.lr_gate_bwd(x, np.zeros((H, dx)), 2.0, deta, lib=lib)
    want = np.zeros((H, dx))
    for h in range(H):
        for b in range(B):
            for t in range(T):
                want[h] += 0.5 * deta[b, h, t] * x[b, t]
    assert np.abs(dth - want).max() < 1e-14 and np.abs(dxo).max() == 0.0


PINS = [
    pin_linear_primal_equals_dual,
    pin_mlp_primal_equals_dual,
    pin_theorem1_linear_attention,
    pin_b1_delta_rule,
    pin_bT_batch_gd,
    pin_eta_zero,
    pin_one_step_is_gradient_step,
    pin_fig4_loss_ratio,
    pin_golden_scalar_examples,
    pin_mlp_one_step_finite_differences,
    pin_mlp_zero_state,
    pin_mlp_w2_zero_kernel_attention,
    pin_mlp_gelu_closed_values,
    pin_ln_primal_equals_dual,
    pin_ln_one_step_finite_differences,
    pin_ln_gamma_zero,
    pin_mlp_ln_primal_equals_dual,
    pin_mlp_ln_one_step_finite_differences,
    pin_mlp_ln_gamma_zero,
    pin_mlp_ln_normalised_outputs,
    pin_ln_scale_covariance,
    pin_ln_normalised_outputs,
    pin_linear_step_replays_scan,
    pin_ln_step_replays_scan,
    pin_mlp_step_replays_scan,
    pin_step_resumes_a_scan_mid_sequence,
    pin_step_golden_scalar_examples,
    pin_linear_bwd_finite_differences,
    pin_linear_bwd_equals_dual_form_adjoint,
    pin_linear_bwd_eta_zero,
    pin_ln_bwd_finite_differences,
    pin_ln_bwd_equals_autograd_of_dual_form,
    pin_ln_bwd_equals_dual_form_adjoint,
    pin_ln_bwd_eta_zero,
    pin_mlp_bwd_finite_differences,
    pin_mlp_bwd_equals_autograd_of_dual_form,
    pin_mlp_bwd_equals_dual_form_adjoint,
    pin_mlp_bwd_eta_zero,
    pin_gate_closed_forms,
    pin_gate_bwd_finite_differences,
    pin_gate_bwd_zero_vector,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.load())


def test_normal_values_fixture():
    """The golden normal-distribution values against Taylor series of erf and exp,
    summed in 40-digit decimal arithmetic (shares nothing with libm or the oracle)."""
    from decimal import Decimal as D, localcontext

    with localcontext() as ctx:
        ctx.prec = 45
        eps = D(10) ** -42

        def series(term0, nxt):
            s, t, n = D(0), term0, 0
            while abs(t) > eps:
                s += t
                n += 1
                t = nxt(t, n)
            return s

        def arctan_inv(m):  # arctan(1/m)
            x = D(1) / m
            return series(x, lambda t, n: -t * x * x * (2 * n - 1) / (2 * n + 1))

        pi = 4 * (4 * arctan_inv(5) - arctan_inv(239))  # Machin's formula

        def erf(x):  # 2/sqrt(pi) sum (-1)^n x^(2n+1) / (n! (2n+1))
            return 2 / pi.sqrt() * series(x, lambda t, n: -t * x * x * (2 * n - 1) / (n * (2 * n + 1)))

        def exp(x):
            return series(D(1), lambda t, n: t * x / n)

        with open(os.path.join(HERE, "golden", "normal_distribution_values.json")) as f:
            g = json.load(f)
        for s in ("1", "2"):
            a = D(s)
            Phi = (1 + erf(a / D(2).sqrt())) / 2
            phi = exp(-a * a / 2) / (2 * pi).sqrt()
            assert abs(Phi - D(g["Phi"][s])) < D("1e-19"), (s, Phi)
            assert abs(phi - D(g["phi"][s])) < D("1e-19"), (s, phi)
        assert abs((2 / pi).sqrt() - D(g["sqrt_2_over_pi"])) < D("1e-19")


# ---------------------------------------------------------------------------
# Invariants of the oracle (no second formulation needed).
# ---------------------------------------------------------------------------

def test_linear_homogeneity_and_superposition():
    rng = np.random.default_rng(30)
    q, k, v, eta, w0 = rand_linear(rng, 2, 2, 29, 6)
    z, w = oracle.linear(q, k, v, eta, w0, 8)
    z2, w2 = oracle.linear(q, k, 2 * v, eta, 2 * w0, 8)
    assert np.array_equal(z2, 2 * z) and np.array_equal(w2, 2 * w)  # power of two: exact
    za, wa = oracle.linear(q, k, 0 * v, eta, w0, 8)
    zb, wb = oracle.linear(q, k, v, eta, 0 * w0, 8)
    assert rel(za + zb, z) < 1e-13 and rel(wa + wb, w) < 1e-13


def test_chunked_scan_reading_in_fp64():
    """The chunked scan's decomposition, on the oracle: with b | chunk length,
    each chunk's end state is W_start M + C with M its run from the identity
    with v = 0 and C its run from zero; chaining the maps gives every chunk's
    start state, and running the chunks from those states reproduces the
    whole sequence's outputs and end state."""
    rng = np.random.default_rng(35)
    B, H, T, d, b, P = 1, 2, 96, 5, 4, 3
    q, k, v, eta, w0 = rand_linear(rng, B, H, T, d)
    z, w = oracle.linear(q, k, v, eta, w0, b)
    Tc = T // P
    sl = lambda a, p: a[:, :, p * Tc:(p + 1) * Tc]
    eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    W = np.broadcast_to(w0, (B, H, d, d)).copy()
    zs = []
    for p in range(P):
        _, M = oracle.linear(sl(q, p), sl(k, p), 0 * sl(v, p), sl(eta, p), eye, b)
        _, C = oracle.linear(sl(q, p), sl(k, p), sl(v, p), sl(eta, p), 0 * eye, b)
        zp, wp = oracle.linear(sl(q, p), sl(k, p), sl(v, p), sl(eta, p), W, b)
        zs.append(zp)
        assert rel(W @ M + C, wp) < 1e-12
        W = wp
    assert rel(np.concatenate(zs, axis=2), z) < 1e-12 and rel(W, w) < 1e-12


def test_chunked_backward_reading_in_fp64():
    """The chunked backward's decomposition, on the oracle: walking a chunk
    backward from end adjoint E gives start adjoint E M^T + C', with M the
    chunk's forward run from the identity with v = 0 (each mini-batch's
    factor I - 2 K diag(eta) K^T is symmetric) and C' its backward from a zero
    end adjoint; chaining from dW_T over the chunks in reverse gives each
    chunk's end adjoint, and the chunks' backward runs from those reproduce
    the whole sequence's gradients."""
    rng = np.random.default_rng(36)
    B, H, T, d, b, P = 1, 2, 96, 5, 4, 3
    q, k, v, eta, w0 = rand_linear(rng, B, H, T, d)
    dz = rng.standard_normal(q.shape)
    dwT = rng.standard_normal((B, H, d, d))
    full = oracle.linear_bwd(q, k, v, eta, w0, b, dz, dwT)
    Tc = T // P
    sl = lambda a, p: a[:, :, p * Tc:(p + 1) * Tc]
    eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    starts = [np.broadcast_to(w0, (B, H, d, d)).copy()]  # each chunk's start state
    for p in range(P - 1):
        starts.append(oracle.linear(sl(q, p), sl(k, p), sl(v, p), sl(eta, p), starts[-1], b)[1])
    E, parts = dwT, [None] * P
    for p in reversed(range(P)):
        a = (sl(q, p), sl(k, p), sl(v, p), sl(eta, p))
        _, M = oracle.linear(a[0], a[1], 0 * a[2], a[3], eye, b)
        Cp = oracle.linear_bwd(*a, starts[p], b, sl(dz, p))[4]
        parts[p] = oracle.linear_bwd(*a, starts[p], b, sl(dz, p), E)
        S = E @ np.swapaxes(M, -1, -2) + Cp
        assert rel(S, parts[p][4]) < 1e-12
        E = S
    for i in range(4):
        assert rel(np.concatenate([pp[i] for pp in parts], axis=2), full[i]) < 1e-12
    assert rel(E, full[4]) < 1e-12


def test_linear_row_permutation():
    rng = np.random.default_rng(31)
    q, k, v, eta, w0 = rand_linear(rng, 1, 2, 21, 7)
    p = rng.permutation(7)
    z, w = oracle.linear(q, k, v, eta, w0, 4)
    zp, wp = oracle.linear(q, k, v[..., p], eta, w0[:, p, :], 4)
    assert np.array_equal(zp, z[..., p]) and np.array_equal(wp, w[:, :, p, :])


@pytest.mark.parametrize("kind", ["linear", "mlp"])
def test_state_passing(kind):
    rng = np.random.default_rng(32)
    T, T1, b = 40, 24, 8
    if kind == "linear":
        q, k, v, eta, w0 = rand_linear(rng, 2, 2, T, 5)
        z, w = oracle.linear(q, k, v, eta, w0, b)
        za, wa = oracle.linear(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], eta[:, :, :T1], w0, b)
        zb, wb = oracle.linear(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], eta[:, :, T1:], wa, b)
        assert np.array_equal(np.concatenate([za, zb], axis=2), z) and np.array_equal(wb, w)
    else:
        q, k, v, eta, w1, w2 = rand_mlp(rng, 2, 1, T, 4, 7)
        z, a, c = oracle.mlp(q, k, v, eta, w1, w2, b)
        za, aa, ca = oracle.mlp(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], eta[:, :, :T1], w1, w2, b)
        zb, ab, cb = oracle.mlp(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], eta[:, :, T1:], aa, ca, b)
        assert np.array_equal(np.concatenate([za, zb], axis=2), z)
        assert np.array_equal(ab, a) and np.array_equal(cb, c)


def test_thread_count_is_bit_exact():
    rng = np.random.default_rng(33)
    q, k, v, eta, w0 = rand_linear(rng, 3, 5, 33, 8)
    z1, w1 = oracle.linear(q, k, v, eta, w0, 16, nthreads=1)
    z7, w7 = oracle.linear(q, k, v, eta, w0, 16, nthreads=7)
    assert np.array_equal(z1, z7) and np.array_equal(w1, w7)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(34)
    q, k, v, eta, w0 = rand_linear(rng, 2, 3, 0, 4)
    z, w = oracle.linear(q, k, v, eta, w0, 16)
    assert z.shape == (2, 3, 0, 4) and np.array_equal(w, np.broadcast_to(w0, w.shape))


# ---------------------------------------------------------------------------
# Planted mistakes: each mutated oracle must fail at least one pin.
# ---------------------------------------------------------------------------

MUTATIONS = {
    "drop_factor_2": ("g[i] = 2.0 * (s - vt[i]);", "g[i] = (s - vt[i]);"),
    "update_sign": ("W[i * d + j] -= et * g[i] * kt[j];", "W[i * d + j] += et * g[i] * kt[j];"),
    "output_before_update": ("s += W[i * d + j] * qt[j];", "s += Ws[i * d + j] * qt[j];"),
    "grad_at_current_state": ("s += Ws[i * d + j] * kt[j];", "s += W[i * d + j] * kt[j];"),
    "transposed_state": ("s += Ws[i * d + j] * kt[j];", "s += Ws[j * d + i] * kt[j];"),
    "output_reads_key": ("s += W[i * d + j] * qt[j];", "s += W[i * d + j] * kt[j];"),
    "eta_of_first_token": ("const double et = eta[t];\n      /* G_t", "const double et = eta[m0];\n      /* G_t"),
    "mlp_drop_gelu_grad": ("s->delta[u] = acc * gelu_grad(s->a[u]);", "s->delta[u] = acc;"),
    "mlp_w2_update_sign": ("W2[i * hd + u] -= et * s->e[i] * s->x[u];", "W2[i * hd + u] += et * s->e[i] * s->x[u];"),
    "mlp_backprop_through_current_w2": ("acc += s->W2s[i * hd + u] * s->e[i];", "acc += W2[i * hd + u] * s->e[i];"),
    "mlp_output_from_start_w1": ("acc += W1[u * d + j] * qt[j];", "acc += s->W1s[u * d + j] * qt[j];"),
    "mlp_gelu_scale": ("return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));", "return 0.5 * x * (1.0 + erf(x));"),
    # common-mode GELU mistakes: the value and the derivative carry the same error,
    # so only closed values (not consistency between the two) can reject them
    "mlp_gelu_erf_unscaled_both": [
        ("return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));", "return 0.5 * x * (1.0 + erf(x));"),
        ("return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * pi);",
         "return 0.5 * (1.0 + erf(x)) + x * exp(-x * x) / sqrt(pi);")],
    "mlp_gelu_tanh_form_both": [
        ("return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
         "return 0.5 * x * (1.0 + tanh(sqrt(2.0 / 3.14159265358979323846) * (x + 0.044715 * x * x * x)));"),
        ("return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * pi);",
         "const double c = sqrt(2.0 / pi), th = tanh(c * (x + 0.044715 * x * x * x));\n"
         "  return 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * c * (1.0 + 3.0 * 0.044715 * x * x);")],
    "mlp_gelu_grad_density_unnormalised": (
        "x * exp(-0.5 * x * x) / sqrt(2.0 * pi);", "x * exp(-0.5 * x * x);"),
    "mlp_gelu_grad_density_wrong_width": (
        "x * exp(-0.5 * x * x) / sqrt(2.0 * pi);", "x * exp(-x * x) / sqrt(2.0 * pi);"),
    "mlp_ln_no_residual_in_loss": ("const double resid = kt[i] + beta[i] - vt[i] + gamma[i] * yhat[i];",
                                   "const double resid = beta[i] - vt[i] + gamma[i] * yhat[i];"),
    "mlp_ln_vjp_drops_mean": ("s->e[i] = rs * (s->e[i] - m1s - yhat[i] * m2s);",
                              "s->e[i] = rs * (s->e[i] - yhat[i] * m2s);"),
    "mlp_ln_drop_gelu_grad": ("s->delta[u] = gelu_grad(s->a[u]) * back;", "s->delta[u] = back;"),
    "mlp_ln_output_before_update": ("pre += qt[j] * W1[u * d + j];", "pre += qt[j] * s->W1s[u * d + j];"),
    "mlp_ln_no_residual_in_output": ("z[t * d + i] = gamma[i] * yhat[i] + beta[i] + qt[i];",
                                     "z[t * d + i] = gamma[i] * yhat[i] + beta[i];"),
    "ln_sample_variance": ("  var /= (double)d;", "  var /= (double)(d - 1);"),
    "ln_eps_outside_sqrt": ("1.0 / sqrt(var + eps);", "1.0 / (sqrt(var) + eps);"),
    "ln_drop_mean_term": ("rs * (gy[i] - m1s - yhat[i] * m2s);", "rs * (gy[i] - yhat[i] * m2s);"),
    "ln_drop_projection_term": ("rs * (gy[i] - m1s - yhat[i] * m2s);", "rs * (gy[i] - m1s);"),
    "ln_drop_rs": ("gy[i] = rs * (gy[i] -", "gy[i] = (gy[i] -"),
    "ln_no_residual_in_loss": ("const double f = kt[i] + gamma[i] * yhat[i] + beta[i];",
                               "const double f = gamma[i] * yhat[i] + beta[i];"),
    "ln_no_residual_in_output": ("z[t * d + i] = qt[i] + gamma[i] * yhat[i] + beta[i];",
                                 "z[t * d + i] = gamma[i] * yhat[i] + beta[i];"),
    "ln_no_gamma_in_vjp": ("gy[i] = 2.0 * gamma[i] * (f - vt[i]);", "gy[i] = 2.0 * (f - vt[i]);"),
    "ln_output_before_update": ("acc += W[i * d + j] * qt[j];", "acc += Ws[i * d + j] * qt[j];"),
    "ln_grad_at_current_state": ("acc += Ws[i * d + j] * kt[j];", "acc += W[i * d + j] * kt[j];"),
    "step_no_gradient_point_reset": (
        "if (pos[bi] % b == 0) memcpy(Wg, W, sizeof(double) * (size_t)(d * d));\n    /* gradient of",
        "/* gradient of"),
    "step_grad_at_current_state": ("pk += Wg[i * d + j] * ku[j];\n      gr[i]",
                                   "pk += W[i * d + j] * ku[j];\n      gr[i]"),
    "step_output_from_gradient_point": ("zq += W[i * d + j] * qu[j];\n      z[u * d + i] = zq;",
                                        "zq += Wg[i * d + j] * qu[j];\n      z[u * d + i] = zq;"),
    "step_gradient_point_every_token": ("if (pos[bi] % b == 0) memcpy(Wg, W, sizeof(double) * (size_t)(d * d));\n    /* gradient of",
                                        "memcpy(Wg, W, sizeof(double) * (size_t)(d * d));\n    /* gradient of"),
    "ln_step_no_projection_term": ("const double dy = rs * (gy[i] - mg - yh[i] * mgy);",
                                   "const double dy = rs * (gy[i] - mg);"),
    "ln_step_no_residual_in_output": ("z[u * d + i] = qu[i] + ga[i] * yh[i] + be[i];",
                                      "z[u * d + i] = ga[i] * yh[i] + be[i];"),
    "mlp_step_backprop_through_current_w2": ("bp += W2g[i * hd + h] * e[i];",
                                             "bp += W2[i * hd + h] * e[i];"),
    "mlp_step_w1_gradient_point_not_reset": ("memcpy(W1g, W1, sizeof(double) * (size_t)(hd * d));", ""),
    "bwd_gradient_point_adjoint_dropped": ("        A[e] += Ag[e];\n", ""),
    "bwd_eta_sign": ("      gb[i] = -eta[t] * s;", "      gb[i] = eta[t] * s;"),
    "bwd_dq_untransposed": ("for (long i = 0; i < d; ++i) s += Wn[i * d + j] * zt[i];",
                            "for (long i = 0; i < d; ++i) s += Wn[j * d + i] * zt[i];"),
    "bwd_dk_drops_gradient_point_term": ("dk[t * d + j] = -eta[t] * s1 + 2.0 * s2;",
                                         "dk[t * d + j] = -eta[t] * s1;"),
    "gate_sign": ("eta_base / (1.0 + exp(-a));", "eta_base / (1.0 + exp(a));"),
    "gate_no_base": ("eta_base / (1.0 + exp(-a));", "1.0 / (1.0 + exp(-a));"),
    "gate_theta_of_head_0": ("*th = theta + (size_t)h * (size_t)dx;", "*th = theta;"),
    "gate_token_major_output": ("eta[((size_t)bi * (size_t)H + (size_t)h) * (size_t)T + (size_t)t]",
                                "eta[((size_t)bi * (size_t)T + (size_t)t) * (size_t)H + (size_t)h]"),
    "gate_first_token_only": ("+ (size_t)t) * (size_t)dx;", ") * (size_t)dx;"),
    "gate_bwd_no_one_minus_sigmoid": ("eta_base * sg * (1.0 - sg);", "eta_base * sg;"),
    "gate_bwd_dx_from_head_0": ("gx[i] += da * th[i];", "gx[i] += da * theta[i];"),
    "gate_bwd_dtheta_from_first_token": ("+= da * xt[i];", "+= da * x[i];"),
    "gate_bwd_no_base": ("deta[gi] * eta_base * sg", "deta[gi] * sg"),
    "ln_bwd_drop_rs_adjoint": ("drs += ddy[i] * (g[i] - gbar - yh[i] * m);", ""),
    "ln_bwd_drop_mean_adjoint": ("+ dm / (double)d * yh[i] + dgbar / (double)d; /* m, gbar */",
                                 "+ dm / (double)d * yh[i]; /* m, gbar */"),
    "ln_bwd_variance_factor": ("dc[i] += 2.0 / (double)d * c[i] * dvar;",
                               "dc[i] += 1.0 / (double)d * c[i] * dvar;"),
    "ln_bwd_no_residual_in_dq": ("double acc = zt[j]; /* the residual q */",
                                 "double acc = 0.0; /* the residual q */"),
    "ln_bwd_gamma_from_f_only": ("dgam[i] += 2.0 * r[i] * dg[i] + yh[i] * dr;",
                                 "dgam[i] += yh[i] * dr;"),
    "ln_bwd_dk_through_current_state": ("for (long i = 0; i < d; ++i) acc += P[i * d + j] * dyv[i];",
                                        "for (long i = 0; i < d; ++i) acc += N[i * d + j] * dyv[i];"),
    "mlp_bwd_drop_gelu_second_derivative": ("da[u] = ddl[u] * s[u] * gelu_grad2(a[u]);",
                                            "da[u] = 0.0;"),
    "mlp_bwd_gelu_second_derivative_form": ("* (2.0 - x * x);", "* (1.0 - x * x);"),
    "mlp_bwd_gradient_point_adjoint_dropped": ("        A1[i] += G1[i];\n        A2[i] += G2[i];\n", ""),
    "mlp_bwd_dk_through_current_state": ("for (long u = 0; u < hd; ++u) acc += P1[u * d + j] * da[u];",
                                         "for (long u = 0; u < hd; ++u) acc += N1[u * d + j] * da[u];"),
    "mlp_bwd_dq_through_start_state": ("for (long u = 0; u < hd; ++u) acc += N1[u * d + j] * daq[u];",
                                       "for (long u = 0; u < hd; ++u) acc += P1[u * d + j] * daq[u];"),
    "mlp_bwd_eta_sign": ("    deta[t] = dsum;", "    deta[t] = -dsum;"),
    "mlp_bwd_dv_sign": ("dv[t * d + i] = -2.0 * de[i];", "dv[t * d + i] = 2.0 * de[i];"),
    "mlp_bwd_y_adjoint_factor": ("G2[i * hd + u] += 2.0 * de[i] * x[u];", "G2[i * hd + u] += de[i] * x[u];"),
    "bwd_output_adjoint_dropped": ("A[i * d + j] += zt[i] * qt[j];\n    /* W_t",
                                   "A[i * d + j] += 0.0 * zt[i] * qt[j];\n    /* W_t"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    edits = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ttt_oracle.c")).read()
    for old, new in (edits if isinstance(edits, list) else [edits]):
        assert src.count(old) == 1, f"mutation anchor for {name} not unique"
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mut.c")
        with open(path, "w") as f:
            f.write(src)
        lib = oracle.load(oracle.build(path, os.path.join(tmp, "libmut.so")))
        caught = []
        for pin in PINS:
            try:
                with np.errstate(all="ignore"):
                    pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin rejects the planted mistake {name}"
