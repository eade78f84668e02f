"""fp64 primal TTT oracle (ctypes wrapper around ``ttt_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and
by the CPU-baseline leg of the benchmark, never by the product path.  It shares
no code with the HIP kernels.

The C file computes the sequential primal mini-batch TTT forward (and its
one-token decode step, §6.11) of
"论文速览 | TTT" (equinox-blog close reading of "Learning to (Learn at Test
Time)"): §3.1 (update, then output), §3.3 (multi-view loss
||f(k;W) - v||^2, output f(q; W_t)), §3.5 (mini-batch gradient point),
§4.4 (TTT-Linear f = Wx, TTT-MLP f = W2 GELU(W1 x)), §4.6 (per-token eta).

Parity pins live in ``tests/test_oracle_pins.py``.  The GELU form (exact erf,
x Phi(x)) is a reading, since the pages name GELU without a form; its values and
derivative are pinned there to closed normal-distribution values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-std=c99"]


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle C file into a shared library with gcc."""
    tmp = f"{out}.{os.getpid()}.tmp"  # per process: concurrent builders never share it
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    L, I = ctypes.c_long, ctypes.c_int
    lib.ttt_oracle_linear.argtypes = [dp, dp, dp, dp, dp, I, L, L, L, L, L, dp, dp, I]
    lib.ttt_oracle_linear.restype = I
    lib.ttt_oracle_mlp.argtypes = [dp, dp, dp, dp, dp, dp, I, L, L, L, L, L, L, dp, dp, dp, I]
    lib.ttt_oracle_mlp.restype = I
    D = ctypes.c_double
    lib.ttt_oracle_linear_ln.argtypes = [dp, dp, dp, dp, dp, I, dp, dp, D, L, L, L, L, L, dp, dp, I]
    lib.ttt_oracle_linear_ln.restype = I
    lib.ttt_oracle_mlp_ln.argtypes = [dp, dp, dp, dp, dp, dp, I, dp, dp, D, L, L, L, L, L, L, dp, dp,
                                      dp, I]
    lib.ttt_oracle_mlp_ln.restype = I
    ip = ctypes.POINTER(ctypes.c_int)
    lib.ttt_oracle_linear_step.argtypes = [dp, dp, dp, dp, dp, dp, ip, L, L, L, L, dp]
    lib.ttt_oracle_linear_step.restype = I
    lib.ttt_oracle_linear_ln_step.argtypes = [dp, dp, dp, dp, dp, dp, ip, dp, dp, D, L, L, L, L, dp]
    lib.ttt_oracle_linear_ln_step.restype = I
    lib.ttt_oracle_mlp_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ip, L, L, L, L, L, dp]
    lib.ttt_oracle_mlp_step.restype = I
    lib.ttt_oracle_linear_bwd.argtypes = [dp, dp, dp, dp, dp, I, L, L, L, L, L, dp, dp, dp, dp, dp,
                                          dp, dp]
    lib.ttt_oracle_linear_bwd.restype = I
    lib.ttt_oracle_linear_ln_bwd.argtypes = [dp, dp, dp, dp, dp, I, dp, dp, D, L, L, L, L, L, dp,
                                             dp, dp, dp, dp, dp, dp, dp, dp]
    lib.ttt_oracle_linear_ln_bwd.restype = I
    lib.ttt_oracle_mlp_bwd.argtypes = [dp, dp, dp, dp, dp, dp, I, L, L, L, L, L, L, dp, dp, dp,
                                       dp, dp, dp, dp, dp, dp]
    lib.ttt_oracle_mlp_bwd.restype = I
    lib.ttt_oracle_lr_gate.argtypes = [dp, dp, D, L, L, L, L, dp]
    lib.ttt_oracle_lr_gate.restype = I
    lib.ttt_oracle_lr_gate_bwd.argtypes = [dp, dp, D, dp, L, L, L, L, dp, dp]
    lib.ttt_oracle_lr_gate_bwd.restype = I
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if it is absent or stale)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_threads() -> int:
    """Threads for the oracle: every core of the affinity set, at most 16 (the
    host share of one GPU on a shared machine)."""
    return max(1, min(16, host_cores()))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def linear(q, k, v, eta, w0, b: int, nthreads: int | None = None, lib=None):
    """TTT-Linear primal forward.

    q, k, v: [B, H, T, d]; eta: [B, H, T]; w0: [H, d, d] (shared over the
    batch) or [B, H, d, d] (one initial state per unit).
    Returns (z [B, H, T, d], w_T [B, H, d, d]) in float64.
    """
    q, k, v, eta, w0 = map(_f64, (q, k, v, eta, w0))
    B, H, T, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and eta.shape == (B, H, T)
    per_batch = 1 if w0.ndim == 4 else 0
    assert w0.shape == ((B, H, d, d) if per_batch else (H, d, d))
    z = np.zeros((B, H, T, d))
    w_out = np.zeros((B, H, d, d))
    lib = lib or load()
    rc = lib.ttt_oracle_linear(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch,
                               B, H, T, d, int(b), _ptr(z), _ptr(w_out),
                               nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_linear failed with status {rc}")
    return z, w_out


def mlp(q, k, v, eta, w1_0, w2_0, b: int, nthreads: int | None = None, lib=None):
    """TTT-MLP primal forward, f(x) = W2 GELU(W1 x).

    w1_0: [H, hidden, d] or [B, H, hidden, d]; w2_0: [H, d, hidden] or
    [B, H, d, hidden].  Returns (z, w1_T, w2_T) in float64.
    """
    q, k, v, eta, w1_0, w2_0 = map(_f64, (q, k, v, eta, w1_0, w2_0))
    B, H, T, d = q.shape
    per_batch = 1 if w1_0.ndim == 4 else 0
    hidden = w1_0.shape[-2]
    assert w1_0.shape == ((B, H, hidden, d) if per_batch else (H, hidden, d))
    assert w2_0.shape == ((B, H, d, hidden) if per_batch else (H, d, hidden))
    z = np.zeros((B, H, T, d))
    w1 = np.zeros((B, H, hidden, d))
    w2 = np.zeros((B, H, d, hidden))
    lib = lib or load()
    rc = lib.ttt_oracle_mlp(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_0), _ptr(w2_0),
                            per_batch, B, H, T, d, hidden, int(b), _ptr(z), _ptr(w1), _ptr(w2),
                            nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_mlp failed with status {rc}")
    return z, w1, w2


def linear_ln(q, k, v, eta, w0, gamma, beta, eps: float, b: int, nthreads: int | None = None,
              lib=None):
    """TTT-Linear with the LayerNorm + residual inner model, primal forward:
    f(x) = x + gamma * (Wx - mean) / sqrt(var + eps) + beta over the d output
    components of each token.

    gamma, beta: [H, d] (per head).  Other arguments as for ``linear``.
    Returns (z [B, H, T, d], w_T [B, H, d, d]) in float64.
    """
    q, k, v, eta, w0, gamma, beta = map(_f64, (q, k, v, eta, w0, gamma, beta))
    B, H, T, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and eta.shape == (B, H, T)
    assert gamma.shape == (H, d) and beta.shape == (H, d)
    per_batch = 1 if w0.ndim == 4 else 0
    assert w0.shape == ((B, H, d, d) if per_batch else (H, d, d))
    z = np.zeros((B, H, T, d))
    w_out = np.zeros((B, H, d, d))
    lib = lib or load()
    rc = lib.ttt_oracle_linear_ln(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch,
                                  _ptr(gamma), _ptr(beta), float(eps), B, H, T, d, int(b),
                                  _ptr(z), _ptr(w_out), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_linear_ln failed with status {rc}")
    return z, w_out


def mlp_ln(q, k, v, eta, w1_0, w2_0, gamma, beta, eps: float, b: int,
           nthreads: int | None = None, lib=None):
    """TTT-MLP with the LayerNorm + residual wrapper, primal forward:
    f(x) = x + gamma * (y - mean) / sqrt(var + eps) + beta with
    y = W2 GELU(W1 x), over the d output components of each token.

    gamma, beta: [H, d] (per head).  Other arguments as for ``mlp``.
    Returns (z, w1_T, w2_T) in float64.
    """
    q, k, v, eta, w1_0, w2_0, gamma, beta = map(_f64, (q, k, v, eta, w1_0, w2_0, gamma, beta))
    B, H, T, d = q.shape
    per_batch = 1 if w1_0.ndim == 4 else 0
    hidden = w1_0.shape[-2]
    assert w1_0.shape == ((B, H, hidden, d) if per_batch else (H, hidden, d))
    assert w2_0.shape == ((B, H, d, hidden) if per_batch else (H, d, hidden))
    assert gamma.shape == (H, d) and beta.shape == (H, d)
    z = np.zeros((B, H, T, d))
    w1 = np.zeros((B, H, hidden, d))
    w2 = np.zeros((B, H, d, hidden))
    lib = lib or load()
    rc = lib.ttt_oracle_mlp_ln(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_0), _ptr(w2_0),
                               per_batch, _ptr(gamma), _ptr(beta), float(eps), B, H, T, d, hidden,
                               int(b), _ptr(z), _ptr(w1), _ptr(w2), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_mlp_ln failed with status {rc}")
    return z, w1, w2


def _ipos(pos, B) -> np.ndarray:
    p = np.ascontiguousarray(np.asarray(pos, dtype=np.int32))
    assert p.shape == (B,) and (p >= 0).all()
    return p


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def linear_step(q, k, v, eta, w, wg, pos, b: int, lib=None):
    """One TTT-Linear decode step (primal form) for every (batch, head) unit.

    q, k, v: [B, H, d] (this token's views); eta: [B, H]; w, wg: [B, H, d, d],
    the current state and the gradient point (the state at the start of the
    current mini-batch); pos: [B] token index of this token (the step sets
    wg = w first when pos % b == 0).  Inputs are not modified.
    Returns (z [B, H, d], w_new, wg_new) in float64.
    """
    q, k, v, eta = map(_f64, (q, k, v, eta))
    B, H, d = q.shape
    w, wg = _f64(w).copy(), _f64(wg).copy()
    assert w.shape == (B, H, d, d) and wg.shape == w.shape and eta.shape == (B, H)
    p = _ipos(pos, B)
    z = np.zeros((B, H, d))
    lib = lib or load()
    rc = lib.ttt_oracle_linear_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w), _ptr(wg),
                                    _iptr(p), B, H, d, int(b), _ptr(z))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_linear_step failed with status {rc}")
    return z, w, wg


def linear_ln_step(q, k, v, eta, w, wg, pos, gamma, beta, eps: float, b: int, lib=None):
    """One decode step of TTT-Linear with the LayerNorm + residual inner
    model; arguments as for ``linear_step`` plus gamma, beta [H, d] and eps."""
    q, k, v, eta, gamma, beta = map(_f64, (q, k, v, eta, gamma, beta))
    B, H, d = q.shape
    w, wg = _f64(w).copy(), _f64(wg).copy()
    assert w.shape == (B, H, d, d) and wg.shape == w.shape and gamma.shape == (H, d)
    p = _ipos(pos, B)
    z = np.zeros((B, H, d))
    lib = lib or load()
    rc = lib.ttt_oracle_linear_ln_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w), _ptr(wg),
                                       _iptr(p), _ptr(gamma), _ptr(beta), float(eps), B, H, d,
                                       int(b), _ptr(z))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_linear_ln_step failed with status {rc}")
    return z, w, wg


def mlp_step(q, k, v, eta, w1, w2, w1g, w2g, pos, b: int, lib=None):
    """One TTT-MLP decode step: w1, w1g [B, H, hidden, d]; w2, w2g
    [B, H, d, hidden].  Returns (z, w1_new, w2_new, w1g_new, w2g_new)."""
    q, k, v, eta = map(_f64, (q, k, v, eta))
    B, H, d = q.shape
    w1, w2, w1g, w2g = (_f64(a).copy() for a in (w1, w2, w1g, w2g))
    hidden = w1.shape[-2]
    assert w1.shape == (B, H, hidden, d) and w2.shape == (B, H, d, hidden)
    assert w1g.shape == w1.shape and w2g.shape == w2.shape
    p = _ipos(pos, B)
    z = np.zeros((B, H, d))
    lib = lib or load()
    rc = lib.ttt_oracle_mlp_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1), _ptr(w2),
                                 _ptr(w1g), _ptr(w2g), _iptr(p), B, H, d, hidden, int(b), _ptr(z))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_mlp_step failed with status {rc}")
    return z, w1, w2, w1g, w2g


def linear_bwd(q, k, v, eta, w0, b: int, dz, dw_T=None, lib=None):
    """Backward of the TTT-Linear scan (reverse pass of the primal form):
    given dz [B, H, T, d] (adjoint of Z) and optionally dw_T [B, H, d, d]
    (adjoint of the final state), returns (dq, dk, dv, deta, dw0) with dw0
    per unit [B, H, d, d] (sum over the batch for a shared initial state).
    """
    q, k, v, eta, w0, dz = map(_f64, (q, k, v, eta, w0, dz))
    B, H, T, d = q.shape
    per_batch = 1 if w0.ndim == 4 else 0
    assert w0.shape == ((B, H, d, d) if per_batch else (H, d, d)) and dz.shape == q.shape
    dwT = None if dw_T is None else _f64(dw_T)
    dq, dk, dv = (np.zeros((B, H, T, d)) for _ in range(3))
    deta = np.zeros((B, H, T))
    dw0 = np.zeros((B, H, d, d))
    lib = lib or load()
    rc = lib.ttt_oracle_linear_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch,
                                   B, H, T, d, int(b), _ptr(dz),
                                   None if dwT is None else _ptr(dwT), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(deta), _ptr(dw0))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_linear_bwd failed with status {rc}")
    return dq, dk, dv, deta, dw0


def linear_ln_bwd(q, k, v, eta, w0, gamma, beta, eps: float, b: int, dz, dw_T=None, lib=None):
    """Backward of TTT-Linear with the LayerNorm + residual inner model:
    given dz [B, H, T, d] and optionally dw_T [B, H, d, d], returns (dq, dk,
    dv, deta, dw0, dgamma, dbeta) with dw0 [B, H, d, d] and dgamma, dbeta
    [B, H, d] per unit (sum over the batch for the shared parameters)."""
    q, k, v, eta, w0, gamma, beta, dz = map(_f64, (q, k, v, eta, w0, gamma, beta, dz))
    B, H, T, d = q.shape
    per_batch = 1 if w0.ndim == 4 else 0
    assert w0.shape == ((B, H, d, d) if per_batch else (H, d, d)) and dz.shape == q.shape
    assert gamma.shape == (H, d) and beta.shape == (H, d)
    dwT = None if dw_T is None else _f64(dw_T)
    dq, dk, dv = (np.zeros((B, H, T, d)) for _ in range(3))
    deta = np.zeros((B, H, T))
    dw0 = np.zeros((B, H, d, d))
    dg, db = np.zeros((B, H, d)), np.zeros((B, H, d))
    lib = lib or load()
    rc = lib.ttt_oracle_linear_ln_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch,
                                      _ptr(gamma), _ptr(beta), float(eps), B, H, T, d, int(b),
                                      _ptr(dz), None if dwT is None else _ptr(dwT), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0), _ptr(dg), _ptr(db))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_linear_ln_bwd failed with status {rc}")
    return dq, dk, dv, deta, dw0, dg, db


def mlp_bwd(q, k, v, eta, w1_0, w2_0, b: int, dz, dw1_T=None, dw2_T=None, lib=None):
    """Backward of the TTT-MLP scan (reverse pass of the primal form): given
    dz [B, H, T, d] and optionally the adjoints of the final states dw1_T
    [B, H, hidden, d], dw2_T [B, H, d, hidden], returns (dq, dk, dv, deta,
    dw1_0, dw2_0) with the initial-state adjoints per unit."""
    q, k, v, eta, w1_0, w2_0, dz = map(_f64, (q, k, v, eta, w1_0, w2_0, dz))
    B, H, T, d = q.shape
    per_batch = 1 if w1_0.ndim == 4 else 0
    hidden = w1_0.shape[-2]
    assert w1_0.shape == ((B, H, hidden, d) if per_batch else (H, hidden, d))
    assert w2_0.shape == ((B, H, d, hidden) if per_batch else (H, d, hidden)) and dz.shape == q.shape
    d1 = None if dw1_T is None else _f64(dw1_T)
    d2 = None if dw2_T is None else _f64(dw2_T)
    dq, dk, dv = (np.zeros((B, H, T, d)) for _ in range(3))
    deta = np.zeros((B, H, T))
    dw1 = np.zeros((B, H, hidden, d))
    dw2 = np.zeros((B, H, d, hidden))
    lib = lib or load()
    rc = lib.ttt_oracle_mlp_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_0), _ptr(w2_0),
                                per_batch, B, H, T, d, hidden, int(b), _ptr(dz),
                                None if d1 is None else _ptr(d1), None if d2 is None else _ptr(d2),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw1), _ptr(dw2))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_mlp_bwd failed with status {rc}")
    return dq, dk, dv, deta, dw1, dw2


def lr_gate(x, theta_lr, eta_base: float, lib=None):
    """Learnable inner learning rate ("论文速览 | TTT", §4.6): x [B, T, dx]
    layer-input tokens, theta_lr [H, dx] one gate vector per head ->
    eta [B, H, T] = eta_base * sigmoid(theta_lr[h] . x[b, t])."""
    x, th = _f64(x), _f64(theta_lr)
    B, T, dx = x.shape
    H = th.shape[0]
    assert th.shape == (H, dx)
    eta = np.zeros((B, H, T))
    lib = lib or load()
    rc = lib.ttt_oracle_lr_gate(_ptr(x), _ptr(th), float(eta_base), B, T, H, dx, _ptr(eta))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_lr_gate failed with status {rc}")
    return eta


def linear_gated(q, k, v, x, theta_lr, eta_base: float, w0, b: int, nthreads: int | None = None,
                 lib=None):
    """TTT-Linear scan with the gated learning rate: the gate above, then
    the scan with that eta.  Returns (z, w_T, eta)."""
    eta = lr_gate(x, theta_lr, eta_base, lib=lib)
    z, w = linear(q, k, v, eta, w0, b, nthreads=nthreads, lib=lib)
    return z, w, eta


def lr_gate_bwd(x, theta_lr, eta_base: float, deta, lib=None):
    """Backward of lr_gate: deta [B, H, T] (dL/deta) -> (dtheta_lr [H, dx],
    dx [B, T, dx])."""
    x, th, de = _f64(x), _f64(theta_lr), _f64(deta)
    B, T, dx = x.shape
    H = th.shape[0]
    assert th.shape == (H, dx) and de.shape == (B, H, T)
    dth = np.zeros((H, dx))
    dxo = np.zeros((B, T, dx))
    lib = lib or load()
    rc = lib.ttt_oracle_lr_gate_bwd(_ptr(x), _ptr(th), float(eta_base), _ptr(de), B, T, H, dx,
                                    _ptr(dth), _ptr(dxo))
    if rc != 0:
        raise RuntimeError(f"ttt_oracle_lr_gate_bwd failed with status {rc}")
    return dth, dxo
