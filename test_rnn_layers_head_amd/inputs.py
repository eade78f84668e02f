"""Seeded synthetic inputs for the TTT forward scan.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the scan's arithmetic, and it is the one module that both the
oracle tests and the HIP path use.

The pages train on Pile / Books3 activations, which are not available here;
these draws stand in for them with the shapes of the paper's 125M and 1.3B
layers (d = 64 heads) at 2k / 8k / 32k contexts and b = 16 mini-batches
("论文速览 | TTT", §3.5 and §5).

Recipe (per workload):
  * numpy ``default_rng(seed)`` (PCG64), every draw in float64, in the order
    Q, K, V, eta, then the initial state(s);
  * Q, K, V ~ N(0, 1/d) i.i.d. per element, except the drifting long-context
    workload where K and V follow x_1 = e_1, x_t = 0.9 x_{t-1} + sqrt(0.19) e_t
    with e ~ N(0, 1/d) independent per (batch, head, dim, tensor);
  * eta_t = eta_scale * sigmoid(N(0, 1)) per (batch, head, token), or
    U(0, 0.1) for the small fp32 workload; eta_scale = 0.1 except for the
    LayerNorm workloads (0.02, see below);
  * W0 ~ N(0, w_scale^2) per head ([H, d, d]), w_scale = 0.02 except for the
    LayerNorm workloads; TTT-MLP: W1 [H, 4d, d] and W2 [H, d, 4d] from the
    same distribution;
  * LayerNorm + residual inner model (kind "linear_ln"): then
    ln_gamma = 1 + 0.2 N(0, 1) and ln_beta = 0.1 N(0, 1) per (head, dim),
    eps = 1e-5.  W0 uses w_scale = 1/sqrt(d) and eta_scale = 0.02: the
    LayerNorm divides by the spread of W0 k, so the gradient scales like
    1 / |W0| and the step is stable only for eta |k|^2 / var(W0 k) of order
    one (with W0 ~ N(0, 0.02^2) it would be ~40 times larger);
  * TTT-MLP with the same wrapper (kind "mlp_ln"): W1, W2 as for TTT-MLP with
    w_scale = 2/sqrt(d) and eta_scale = 0.01, then ln_gamma, ln_beta as
    above.  With the plain MLP's 0.02 and 0.1 the states grow ~30 times over
    2k tokens; with w_scale = 1/sqrt(d), eta_scale = 0.02 they stay bounded
    but the recurrence is chaotic (a float32 evaluation drifts from a
    float64 one by 0.14 rel-L2 after 2k tokens, doubling every ~50 tokens),
    and at 2/sqrt(d), 0.02 some units still are; with these scales the drift
    is 5e-7 on every unit while W1 moves by a third over the sequence;
  * learning-rate gate workloads (gate_dx > 0), drawn last: the layer input
    x ~ N(0, 1) per element, [B, T, gate_dx], stored bf16, and one gate
    vector per head theta_lr ~ N(0, 1 / gate_dx), [H, gate_dx], fp32, with
    eta_base = eta_scale = 0.1: the gate's logit theta_lr . x is then
    ~N(0, 1), so the gated eta has the distribution 0.1 sigmoid(N(0, 1)) of
    the other workloads.  gate_dx is the model width H d (2048 for the 1.3B
    layer, 768 for the 125M one);
  * the drawn float64 values are rounded once, round-to-nearest-even, to the
    storage dtype (bf16 for Q/K/V unless the workload says fp32; eta and the
    states are fp32).  Both sides consume exactly these rounded values.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "linear" | "linear_ln" | "mlp" | "mlp_ln"
    B: int
    H: int
    T: int
    d: int = 64
    b: int = 16
    hidden: int = 0
    qkv_dtype: str = "bf16"  # "bf16" | "f32"
    eta_dist: str = "sigmoid"  # "sigmoid" | "uniform"
    drift: bool = False
    seed: int = 0
    eta_scale: float = 0.1
    w_scale: float = 0.02
    ln_eps: float = 1e-5
    gate_dx: int = 0  # > 0: draw a gate input x [B, T, gate_dx] and theta_lr [H, gate_dx]
    b_sweep: tuple = field(default_factory=tuple)

    @property
    def units(self) -> int:
        return self.B * self.H

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T


WORKLOADS = {
    1: Workload("linear-fp32-T256", "linear", B=1, H=1, T=256, qkv_dtype="f32",
                eta_dist="uniform", seed=1),
    2: Workload("linear-125M-T2048", "linear", B=8, H=12, T=2048, seed=2),
    3: Workload("linear-1.3B-T8192", "linear", B=4, H=32, T=8192, seed=3,
                b_sweep=(1, 4, 16, 64)),
    4: Workload("mlp-125M-T2048", "mlp", B=8, H=12, T=2048, hidden=256, seed=4),
    5: Workload("linear-longctx-T32768", "linear", B=1, H=32, T=32768, drift=True, seed=5),
    6: Workload("linear-ln-1.3B-T8192", "linear_ln", B=4, H=32, T=8192, seed=6, eta_scale=0.02,
                w_scale=0.125),
    7: Workload("linear-ln-125M-T2048", "linear_ln", B=8, H=12, T=2048, seed=7, eta_scale=0.02,
                w_scale=0.125),
    8: Workload("linear-gated-1.3B-T8192", "linear", B=4, H=32, T=8192, seed=8, gate_dx=2048),
    9: Workload("linear-gated-125M-T2048", "linear", B=8, H=12, T=2048, seed=9, gate_dx=768),
    10: Workload("mlp-ln-125M-T2048", "mlp_ln", B=8, H=12, T=2048, hidden=256, seed=10,
                 eta_scale=0.01, w_scale=0.25),
}


def workload(wid: int, **overrides) -> Workload:
    w = WORKLOADS[wid]
    return replace(w, **overrides) if overrides else w


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16.  Values are first rounded to
    float32 (exact for the magnitudes drawn here), then to bf16.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``q, k, v`` are float32 arrays holding exactly the stored values (bf16
    values widened when the storage dtype is bf16); ``q_raw`` etc. are the
    arrays in storage format (uint16 bf16 patterns or float32).
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    eta: np.ndarray
    w0: np.ndarray | None = None
    w1: np.ndarray | None = None
    w2: np.ndarray | None = None
    q_raw: np.ndarray | None = None
    k_raw: np.ndarray | None = None
    v_raw: np.ndarray | None = None
    ln_gamma: np.ndarray | None = None  # [H, d] fp32 (kinds "linear_ln", "mlp_ln")
    ln_beta: np.ndarray | None = None
    gate_x: np.ndarray | None = None  # [B, T, dx] float32 holding the bf16 values
    gate_x_raw: np.ndarray | None = None  # the same as uint16 bf16 patterns
    theta_lr: np.ndarray | None = None  # [H, dx] fp32

    @property
    def eta_base(self) -> float:
        return self.wl.eta_scale

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q_raw, self.k_raw, self.v_raw, self.eta, self.w0, self.w1, self.w2,
                  self.ln_gamma, self.ln_beta, self.gate_x_raw, self.theta_lr):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()

    def units(self, idx) -> "Inputs":
        """Inputs restricted to a list of flat (batch*H + head) unit indices.

        The result has B = 1, H = len(idx) and carries one initial state per
        unit ([1, n, ...] per-batch layout) so that any subset of units can be
        fed to a reference on its own.
        """
        idx = np.asarray(idx)
        B, H = self.wl.B, self.wl.H
        sel = lambda a: a.reshape(B * H, *a.shape[2:])[idx][None]
        heads = idx % H
        st = lambda a: None if a is None else a[heads][None]
        return Inputs(replace(self.wl, B=1, H=len(idx)), sel(self.q), sel(self.k), sel(self.v),
                      sel(self.eta), st(self.w0), st(self.w1), st(self.w2),
                      None if self.q_raw is None else sel(self.q_raw),
                      None if self.k_raw is None else sel(self.k_raw),
                      None if self.v_raw is None else sel(self.v_raw),
                      None if self.ln_gamma is None else self.ln_gamma[heads],
                      None if self.ln_beta is None else self.ln_beta[heads])


def _ar1(rng: np.random.Generator, shape, rho: float = 0.9) -> np.ndarray:
    """AR(1) draws along axis 2 (tokens) with stationary variance 1/d."""
    B, H, T, d = shape
    e = rng.standard_normal(shape) * np.sqrt(1.0 / d)
    x = np.empty(shape)
    x[:, :, 0] = e[:, :, 0]
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, T):
        x[:, :, t] = rho * x[:, :, t - 1] + c * e[:, :, t]
    return x


def make_inputs(wl: Workload | int, seed: int | None = None) -> Inputs:
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    shape = (wl.B, wl.H, wl.T, wl.d)
    sd = np.sqrt(1.0 / wl.d)
    q = rng.standard_normal(shape) * sd
    if wl.drift:
        k = _ar1(rng, shape)
        v = _ar1(rng, shape)
    else:
        k = rng.standard_normal(shape) * sd
        v = rng.standard_normal(shape) * sd
    if wl.eta_dist == "uniform":
        eta = rng.uniform(0.0, 0.1, size=(wl.B, wl.H, wl.T))
    else:
        eta = wl.eta_scale / (1.0 + np.exp(-rng.standard_normal((wl.B, wl.H, wl.T))))
    eta = eta.astype(np.float32)
    w0 = w1 = w2 = gamma = beta = None
    if wl.kind in ("linear", "linear_ln"):
        w0 = (rng.standard_normal((wl.H, wl.d, wl.d)) * wl.w_scale).astype(np.float32)
    elif wl.kind in ("mlp", "mlp_ln"):
        hd = wl.hidden or 4 * wl.d
        w1 = (rng.standard_normal((wl.H, hd, wl.d)) * wl.w_scale).astype(np.float32)
        w2 = (rng.standard_normal((wl.H, wl.d, hd)) * wl.w_scale).astype(np.float32)
    else:
        raise ValueError(wl.kind)
    if wl.kind in ("linear_ln", "mlp_ln"):
        gamma = (1.0 + 0.2 * rng.standard_normal((wl.H, wl.d))).astype(np.float32)
        beta = (0.1 * rng.standard_normal((wl.H, wl.d))).astype(np.float32)
    if wl.qkv_dtype == "bf16":
        raws = [bf16_bits(a) for a in (q, k, v)]
        vals = [bf16_to_f32(r) for r in raws]
    elif wl.qkv_dtype == "f32":
        vals = [a.astype(np.float32) for a in (q, k, v)]
        raws = vals
    else:
        raise ValueError(wl.qkv_dtype)
    gx = gx_raw = theta = None
    if wl.gate_dx:
        gx_raw = bf16_bits(rng.standard_normal((wl.B, wl.T, wl.gate_dx)))
        gx = bf16_to_f32(gx_raw)
        theta = (rng.standard_normal((wl.H, wl.gate_dx)) / np.sqrt(wl.gate_dx)).astype(np.float32)
    return Inputs(wl, *vals, eta, w0, w1, w2, *raws, gamma, beta, gx, gx_raw, theta)
