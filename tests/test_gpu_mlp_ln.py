"""TTT-MLP with the LayerNorm + residual wrapper, f(x) = x + LN(W2 GELU(W1 x))
("论文速览 | TTT" §4.4 with §3.7), through the C ABI against the fp64 oracle.

bf16 inputs with b | 16 run the dual-form scan (bf16 MFMA on hi + lo
splits, ~2^-16 relative per product), with 16 | b the same scan with the
gradient point held across the mini-batch's tiles; fp32 inputs the primal
form in fp32 arithmetic.  The bound is the LayerNorm bound of the linear wrapper,
rel-L2 <= 1e-4 and max|diff| / RMS <= 1e-3, on z and both final states.  On the 2k-token workload the max bound is
max(1e-3, 1.5 x the fp32 floor).  The floor is what a plain float32
evaluation of the same method (torch on the CPU, the dual form, batched over
the units) reaches against the oracle on the same inputs, computed in the
test (about 5e-6 there).  The workload's scales keep the recurrence
well-conditioned: at W ~ N(0, 1/d) it is chaotic, and no fp32 evaluation
stays near the fp64 oracle past ~1k tokens.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import oracle
from test_rnn_layers_head_amd import TTTError, inputs, ttt_mlp_ln_fwd

pytestmark = pytest.mark.gpu


def case(B, H, T, dtype, seed):
    return inputs.make_inputs(inputs.Workload("mlp-ln-small", "mlp_ln", B=B, H=H, T=T, hidden=256,
                                              qkv_dtype=dtype, seed=seed, eta_scale=0.01,
                                              w_scale=0.25))


def run(x, b, gamma=None, beta=None, eps=None):
    gamma = x.ln_gamma if gamma is None else gamma
    beta = x.ln_beta if beta is None else beta
    eps = x.wl.ln_eps if eps is None else eps
    out = ttt_mlp_ln_fwd(gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"), gu.f32(x.eta),
                         gu.f32(x.w1), gu.f32(x.w2), gu.f32(gamma), gu.f32(beta), eps, b)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def close(got, ref, what, rel=1e-4, mx=1e-3):
    m = gu.metrics(got, ref)
    assert m["rel_l2"] <= rel and m["max_over_rms"] <= mx, (what, m)
    return m


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_small_parity(dtype, b, T):
    x = case(2, 2, T, dtype, seed=1000 + T + b)
    got = run(x, b)
    ref = oracle.mlp_ln(x.q, x.k, x.v, x.eta, x.w1, x.w2, x.ln_gamma, x.ln_beta, x.wl.ln_eps, b)
    out = {n: close(g, r, n)["rel_l2"] for n, g, r in zip(("z", "w1", "w2"), got, ref)}
    print(f"{dtype} T={T} b={b}:", out)


@pytest.mark.parametrize("b", [32, 48, 64])
@pytest.mark.parametrize("T", [16, 130, 200])
def test_held_gradient_point(b, T):
    """Mini-batches of several tiles (bf16): ragged last mini-batch, tile
    counts that are and are not multiples of b / 16."""
    x = case(1, 3, T, "bf16", seed=1100 + T + b)
    got = run(x, b)
    ref = oracle.mlp_ln(x.q, x.k, x.v, x.eta, x.w1, x.w2, x.ln_gamma, x.ln_beta, x.wl.ln_eps, b)
    out = {n: close(g, r, n)["rel_l2"] for n, g, r in zip(("z", "w1", "w2"), got, ref)}
    print(f"bf16 T={T} b={b}:", out)


@pytest.mark.parametrize("dtype, b", [("bf16", 16), ("bf16", 4), ("bf16", 32), ("f32", 16)])
def test_gamma_zero_freezes_the_state(dtype, b):
    """gamma = 0: no gradient passes the LayerNorm, z = q + beta exactly and
    the state is unchanged (both kernels' arithmetic on this path is exact)."""
    x = case(1, 3, 50, dtype, seed=1010)
    z, w1, w2 = run(x, b, gamma=np.zeros_like(x.ln_gamma))
    assert np.array_equal(w1, np.broadcast_to(x.w1, w1.shape))
    assert np.array_equal(w2, np.broadcast_to(x.w2, w2.shape))
    assert np.array_equal(z, (x.q + x.ln_beta[None, :, None, :]).astype(np.float32))


def fp32_floor(x, b=16):
    """z, W1_T, W2_T by a plain float32 evaluation of the dual form ("论文速览 |
    TTT" §3.7 with the §4.4 wrapper), torch on the CPU, batched over units."""
    B, H, T, d = x.q.shape
    U, f, eps = B * H, torch.float32, x.wl.ln_eps
    tt = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=f)
    q, k, v = (tt(a.reshape(U, T, d)) for a in (x.q, x.k, x.v))
    eta = tt(x.eta.reshape(U, T))
    W1 = tt(np.broadcast_to(x.w1, (B, H) + x.w1.shape[1:]).reshape(U, *x.w1.shape[1:]))
    W2 = tt(np.broadcast_to(x.w2, (B, H) + x.w2.shape[1:]).reshape(U, *x.w2.shape[1:]))
    g_ = tt(np.tile(x.ln_gamma, (B, 1)))[:, :, None]
    b_ = tt(np.tile(x.ln_beta, (B, 1)))[:, :, None]
    gelu = lambda a: 0.5 * a * (1.0 + torch.erf(a / np.sqrt(2.0)))
    dgelu = lambda a: 0.5 * (1.0 + torch.erf(a / np.sqrt(2.0))) + a * torch.exp(-0.5 * a * a) / np.sqrt(2 * np.pi)

    def lnhat(Y):
        mu = Y.mean(dim=1, keepdim=True)
        rs = 1.0 / torch.sqrt(((Y - mu) ** 2).mean(dim=1, keepdim=True) + eps)
        return (Y - mu) * rs, rs

    outs = []
    for m0 in range(0, T, b):
        XK, XV, XQ = (a[:, m0:m0 + b].transpose(1, 2) for a in (k, v, q))
        Z1 = W1 @ XK
        X2 = gelu(Z1)
        Yh, rs = lnhat(W2 @ X2)
        g = 2.0 * g_ * (XK + g_ * Yh + b_ - XV)
        G2 = rs * (g - g.mean(dim=1, keepdim=True) - Yh * (g * Yh).mean(dim=1, keepdim=True))
        G2 = G2 * eta[:, m0:m0 + b][:, None, :]
        G1 = (W2.transpose(1, 2) @ G2) * dgelu(Z1)
        X2q = gelu(W1 @ XQ - G1 @ torch.triu(XK.transpose(1, 2) @ XQ))
        Oh, _ = lnhat(W2 @ X2q - G2 @ torch.triu(X2.transpose(1, 2) @ X2q))
        outs.append((XQ + g_ * Oh + b_).transpose(1, 2))
        W1 = W1 - G1 @ XK.transpose(1, 2)
        W2 = W2 - G2 @ X2.transpose(1, 2)
    return [torch.cat(outs, dim=1).numpy(), W1.numpy(), W2.numpy()]


def test_125m_workload_all_units():
    """Every unit of the 125M MLP-LN workload (B8 H12 T2048, b = 16)."""
    x = inputs.make_inputs(10)
    got = run(x, 16)
    assert all(np.isfinite(a).all() for a in got)
    ref = oracle.mlp_ln(x.q, x.k, x.v, x.eta, x.w1, x.w2, x.ln_gamma, x.ln_beta, x.wl.ln_eps, 16)
    floor = fp32_floor(x)
    out = {}
    for name, g, r, fl in zip(("z", "w1", "w2"), got, ref, floor):
        f = gu.metrics(fl.reshape(r.shape), r)["max_over_rms"]
        m = close(g, r, f"125M {name}", rel=1e-4, mx=max(1e-3, 1.5 * f))
        out[name] = (m["rel_l2"], m["max_over_rms"], f)
    print("MLP-LN 125M (rel-L2, max/RMS, fp32 floor max/RMS):", out)


def test_empty_sequence_and_rejected_arguments():
    x = case(1, 2, 16, "bf16", seed=1020)
    e = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    z, w1, w2 = ttt_mlp_ln_fwd(e, e, e, torch.empty(1, 2, 0, device="cuda"), gu.f32(x.w1),
                               gu.f32(x.w2), gu.f32(x.ln_gamma), gu.f32(x.ln_beta), 1e-5, 16)
    torch.cuda.synchronize()
    assert np.array_equal(w1.cpu().numpy(), np.broadcast_to(x.w1, w1.shape))
    args = (gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"), gu.f32(x.eta), gu.f32(x.w1),
            gu.f32(x.w2), gu.f32(x.ln_gamma), gu.f32(x.ln_beta))
    with pytest.raises(TTTError, match="TTT_ERR_VALUE"):
        ttt_mlp_ln_fwd(*args, 0.0, 16)
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_mlp_ln_fwd(*args, 1e-5, 24)
