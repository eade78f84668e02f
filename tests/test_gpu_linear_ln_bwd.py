"""TTT-Linear with the LayerNorm + residual inner model: the forward (the
primal form for fp32 q/k/v), the forward with checkpoints (the dual-form
scan with checkpoint stores for bf16, else the primal form) and the backward
through the scan, through the C ABI, against the fp64 oracle ("论文速览 |
TTT" §4.4, §6.12).

bf16 q/k/v with b | 16 run the dual-form backward (hi + lo splits, ~2^-16
relative per product; b < 16 with one mini-batch per 16-token tile, its
other rows zero tokens), every other case the primal form in fp32
arithmetic.
Tolerance: up to a few hundred tokens the LayerNorm forward bound (rel-L2 <=
1e-4, max|diff| / RMS <= 1e-3) applies to outputs, checkpoints and every
gradient.  Over the
2k-token workload the LayerNorm recurrence amplifies rounding in the adjoint
as it does in the forward: float32 autodiff of the dual form
(``fp32_floor``, computed in the test) reaches max|diff| / RMS = 1.04e-2 on dv
against the fp64 oracle (the dual-form backward from the dual-form
forward's checkpoints: 1.24e-2).  The bound there is rel-L2 <= 2e-3 and max|diff| /
RMS <= max(1e-2, 1.5 x that floor), gradient by gradient.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import oracle
from test_rnn_layers_head_amd import (TTTError, inputs, ttt_linear_ln_bwd, ttt_linear_ln_fwd,
                                      ttt_linear_ln_fwd_ckpt)

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "deta", "dw0", "dgamma", "dbeta")


def close(got, ref, what, rel=1e-4, mx=1e-3):
    m = gu.metrics(got, ref)
    assert m["rel_l2"] <= rel and m["max_over_rms"] <= mx, (what, m)
    return m


def case(B, H, T, dtype, seed):
    return inputs.make_inputs(inputs.Workload("ln-bwd", "linear_ln", B=B, H=H, T=T, qkv_dtype=dtype,
                                              seed=seed, eta_scale=0.02, w_scale=0.125))


def dev_all(x):
    return ((gu.dev(x, n) for n in "qkv"), gu.f32(x.eta), gu.f32(x.w0), gu.f32(x.ln_gamma),
            gu.f32(x.ln_beta))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 8, 16, 32])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_primal_forward_any_minibatch(dtype, b, T):
    """b < 16 or fp32 inputs: the primal-form forward, against the oracle."""
    if dtype == "bf16" and b % 16 == 0:
        pytest.skip("the dual-form kernel (test_gpu_linear_ln.py)")
    x = case(2, 2, T, dtype, seed=900 + T + b)
    z, w = gu.run_linear_ln(x, b)
    zr, wr = gu.oracle_linear_ln(x, b)
    print(f"{dtype} T={T} b={b} z:", close(z, zr, "z"), "w:", close(w, wr, "w_T"))


@pytest.mark.parametrize("with_dwT", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 16, 32])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_backward_parity(with_dwT, dtype, b, T):
    x = case(2, 2, T, dtype, seed=910 + T + b)
    (q, k, v), eta, w0, gam, bet = dev_all(x)
    eps = x.wl.ln_eps
    rng = np.random.default_rng(911 + T)
    dz = rng.standard_normal(x.q.shape).astype(np.float32)
    dwT = rng.standard_normal((2, 2, 64, 64)).astype(np.float32) if with_dwT else None
    z, w, ck = ttt_linear_ln_fwd_ckpt(q, k, v, eta, w0, gam, bet, eps, b)
    g = ttt_linear_ln_bwd(q, k, v, eta, ck, gam, bet, eps, b, gu.f32(dz),
                          None if dwT is None else gu.f32(dwT))
    torch.cuda.synchronize()
    zr, wr = gu.oracle_linear_ln(x, b)
    close(z.cpu().numpy(), zr, "z")
    close(w.cpu().numpy(), wr, "w_T")
    ck = ck.cpu().numpy()
    for m in range(1, ck.shape[2]):
        _, ref = oracle.linear_ln(x.q[:, :, :b * m], x.k[:, :, :b * m], x.v[:, :, :b * m],
                                  x.eta[:, :, :b * m], x.w0, x.ln_gamma, x.ln_beta, eps, b)
        close(ck[:, :, m], ref, f"checkpoint {m}")
    ref = oracle.linear_ln_bwd(x.q, x.k, x.v, x.eta, x.w0, x.ln_gamma, x.ln_beta, eps, b, dz, dwT)
    got = [t.cpu().numpy() for t in g]
    out = {name: close(a, r, f"T={T} b={b} {name}")["rel_l2"] for name, a, r in zip(NAMES, got, ref)}
    print(f"{dtype} T={T} b={b} dW_T={with_dwT}:", out)


@pytest.mark.parametrize("b", [4, 16, 32, 64])
def test_forward_with_checkpoints_matches_plain_forward(b):
    """bf16 with b | 16 or 16 | b: ttt_linear_ln_fwd_ckpt runs the dual-form
    scan of ttt_linear_ln_fwd with checkpoint stores added, so z and the
    final state are bit-identical, and checkpoint 0 is W0 itself."""
    x = case(1, 3, 100, "bf16", seed=930 + b)
    (q, k, v), eta, w0, gam, bet = dev_all(x)
    eps = x.wl.ln_eps
    z0, w1 = ttt_linear_ln_fwd(q, k, v, eta, w0, gam, bet, eps, b)
    z, w, ck = ttt_linear_ln_fwd_ckpt(q, k, v, eta, w0, gam, bet, eps, b)
    torch.cuda.synchronize()
    assert torch.equal(z0, z) and torch.equal(w1, w)
    assert ck.shape[2] == (100 + b - 1) // b
    assert np.array_equal(ck[:, :, 0].cpu().numpy(), np.broadcast_to(x.w0, (1, 3, 64, 64)))


def fp32_floor(x, dz, b=16):
    """Every gradient of <dZ, Z> by torch float32 autodiff of the LayerNorm
    scan's dual form ("论文速览 | TTT" §3.6 with the §4.4 wrapper), batched over
    the units: what fp32 arithmetic alone reaches on this workload."""
    B, H, T, d = x.q.shape
    U, f, eps = B * H, torch.float32, x.wl.ln_eps
    tt = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=f).requires_grad_()
    q, k, v = (tt(a.reshape(U, T, d)) for a in (x.q, x.k, x.v))
    eta = tt(x.eta.reshape(U, T))
    w0 = tt(np.broadcast_to(x.w0, (B, H, d, d)).reshape(U, d, d))
    gam, bet = tt(np.tile(x.ln_gamma, (B, 1))), tt(np.tile(x.ln_beta, (B, 1)))

    def lnhat(Y):
        mu = Y.mean(dim=1, keepdim=True)
        rs = 1.0 / torch.sqrt(((Y - mu) ** 2).mean(dim=1, keepdim=True) + eps)
        return (Y - mu) * rs, rs

    W, g_, b_, outs = w0, gam[:, :, None], bet[:, :, None], []
    for m0 in range(0, T, b):
        XK, XV, XQ = (a[:, m0:m0 + b].transpose(1, 2) for a in (k, v, q))
        Yh, rs = lnhat(W @ XK)
        g = 2.0 * g_ * (XK + g_ * Yh + b_ - XV)
        G = rs * (g - g.mean(dim=1, keepdim=True) - Yh * (g * Yh).mean(dim=1, keepdim=True))
        Ge = G * eta[:, m0:m0 + b][:, None, :]
        outs.append((XQ + g_ * lnhat(W @ XQ - Ge @ torch.triu(XK.transpose(1, 2) @ XQ))[0]
                     + b_).transpose(1, 2))
        W = W - Ge @ XK.transpose(1, 2)
    (torch.cat(outs, dim=1) * torch.tensor(dz.reshape(U, T, d))).sum().backward()
    return [t.grad.numpy() for t in (q, k, v, eta, w0, gam, bet)]


def test_backward_125m_ln_workload_all_units():
    """Every unit of the LayerNorm 125M workload (b = 16) against the oracle
    backward, which runs one unit per call on a thread pool."""
    x = inputs.make_inputs(7)
    (q, k, v), eta, w0, gam, bet = dev_all(x)
    eps = x.wl.ln_eps
    rng = np.random.default_rng(920)
    dz = (rng.standard_normal(x.q.shape) * 0.1).astype(np.float32)
    _, _, ck = ttt_linear_ln_fwd_ckpt(q, k, v, eta, w0, gam, bet, eps, 16)
    got = [t.cpu().numpy() for t in ttt_linear_ln_bwd(q, k, v, eta, ck, gam, bet, eps, 16,
                                                      gu.f32(dz))]
    torch.cuda.synchronize()
    assert all(np.isfinite(a).all() for a in got)
    dzu = dz.reshape(-1, x.wl.T, 64)
    H = x.wl.H

    def one(u):
        s = x.units([u])
        h = u % H
        return oracle.linear_ln_bwd(s.q, s.k, s.v, s.eta, s.w0, x.ln_gamma[h:h + 1],
                                    x.ln_beta[h:h + 1], eps, 16, dzu[u][None, None])

    per = gu.oracle_units_parallel(one, x.wl.units)
    floor = fp32_floor(x, dz)
    out = {}
    for i, name in enumerate(NAMES):
        ref = np.concatenate([p[i] for p in per], axis=1).reshape(got[i].shape)
        fl = gu.metrics(floor[i].reshape(ref.shape), ref)["max_over_rms"]
        m = close(got[i], ref, f"125M {name}", rel=gu.TOL_BF16_REL,
                  mx=max(gu.TOL_BF16_MAX, 1.5 * fl))
        out[name] = (m["rel_l2"], m["max_over_rms"], fl)
    print("LN 125M backward (rel-L2, max/RMS, fp32 floor max/RMS):", out)


def test_backward_empty_sequence_and_rejected_arguments():
    x = case(1, 2, 16, "bf16", seed=930)
    (q, k, v), eta, w0, gam, bet = dev_all(x)
    e = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    dwT = torch.randn(1, 2, 64, 64, device="cuda")
    g = ttt_linear_ln_bwd(e, e, e, torch.empty(1, 2, 0, device="cuda"),
                          torch.empty(1, 2, 0, 64, 64, device="cuda"), gam, bet, 1e-5, 16,
                          torch.empty(1, 2, 0, 64, device="cuda"), dwT)
    torch.cuda.synchronize()
    assert torch.equal(g[4], dwT) and not g[5].any() and not g[6].any()
    _, _, ck = ttt_linear_ln_fwd_ckpt(q, k, v, eta, w0, gam, bet, 1e-5, 16)
    with pytest.raises(TTTError, match="TTT_ERR_VALUE"):
        ttt_linear_ln_bwd(q, k, v, eta, ck, gam, bet, 0.0, 16, torch.randn(1, 2, 16, 64, device="cuda"))
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_linear_ln_fwd(q, k, v, eta, w0, gam, bet, 1e-5, 24)
