"""TTT-MLP training support: the checkpointing forward and the backward through
the scan (through the C ABI) against the fp64 oracle ("论文速览 | TTT" §6.12).

Tolerance: for fp32 inputs the fp32 bound (rel-L2 <= 1e-5) on every
gradient; for bf16 inputs the bf16-input bound of the forward (rel-L2 <= 2e-3,
max|diff| / RMS <= 1e-2), as for the TTT-Linear backward.  bf16 q/k/v with
b = 16 run the dual-form backward (bf16 MFMA on hi + lo splits, ~2^-16
relative per product); other cases the primal backward in fp32 arithmetic.
For bf16 q/k/v with b | 16 the checkpoints come from the bf16 dual-form
forward, for fp32 from the primal fp32 kernel.  The errors are printed.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import oracle
from test_rnn_layers_head_amd import TTTError, inputs, ttt_mlp_bwd, ttt_mlp_fwd, ttt_mlp_fwd_ckpt

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "deta", "dw1_0", "dw2_0")


def case(B, H, T, dtype, seed):
    return inputs.make_inputs(inputs.Workload("mlp-bwd", "mlp", B=B, H=H, T=T, hidden=256,
                                              qkv_dtype=dtype, seed=seed))


def run_fwd_bwd(x, b, dz, dw1=None, dw2=None):
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta = gu.f32(x.eta)
    z, w1, w2, c1, c2 = ttt_mlp_fwd_ckpt(q, k, v, eta, gu.f32(x.w1), gu.f32(x.w2), b)
    g = ttt_mlp_bwd(q, k, v, eta, c1, c2, b, gu.f32(dz), None if dw1 is None else gu.f32(dw1),
                    None if dw2 is None else gu.f32(dw2))
    torch.cuda.synchronize()
    return ([t.cpu().numpy() for t in (z, w1, w2)], [t.cpu().numpy() for t in (c1, c2)],
            [t.cpu().numpy() for t in g])


def check(got, ref, what, dtype="bf16"):
    out = {}
    for name, a, r in zip(NAMES, got, ref):
        out[name] = gu.assert_close(a, r, dtype, f"{what} {name}")["rel_l2"]
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_checkpoints_are_the_states_before_each_minibatch(dtype, b, T):
    x = case(1, 2, T, dtype, seed=800 + T + b)
    rng = np.random.default_rng(801)
    (z, w1, w2), (c1, c2), _ = run_fwd_bwd(x, b, rng.standard_normal(x.q.shape).astype(np.float32))
    zr, w1r, w2r = gu.oracle_mlp(x, b)
    gu.assert_close(z, zr, "bf16", "z")
    gu.assert_close(w1, w1r, "bf16", "w1")
    gu.assert_close(w2, w2r, "bf16", "w2")
    for m in range(c1.shape[2]):
        if m == 0:
            s1, s2 = np.broadcast_to(x.w1, c1[:, :, 0].shape), np.broadcast_to(x.w2, c2[:, :, 0].shape)
        else:
            t1 = m * b
            _, s1, s2 = oracle.mlp(x.q[:, :, :t1], x.k[:, :, :t1], x.v[:, :, :t1], x.eta[:, :, :t1],
                                   x.w1, x.w2, b)
        gu.assert_close(c1[:, :, m], s1, "bf16", f"w1_ckpt[{m}]")
        gu.assert_close(c2[:, :, m], s2, "bf16", f"w2_ckpt[{m}]")


@pytest.mark.parametrize("with_dwT", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 37, 100])
def test_backward_parity(with_dwT, dtype, b, T):
    x = case(2, 2, T, dtype, seed=810 + T + b)
    rng = np.random.default_rng(811 + T)
    dz = rng.standard_normal(x.q.shape).astype(np.float32)
    d1 = rng.standard_normal((2, 2, 256, 64)).astype(np.float32) if with_dwT else None
    d2 = rng.standard_normal((2, 2, 64, 256)).astype(np.float32) if with_dwT else None
    _, _, got = run_fwd_bwd(x, b, dz, d1, d2)
    ref = oracle.mlp_bwd(x.q, x.k, x.v, x.eta, x.w1, x.w2, b, dz, d1, d2)
    print(f"{dtype} T={T} b={b} dW_T={with_dwT}:", check(got, ref, f"T={T} b={b}", dtype))


def test_backward_125m_workload_all_units():
    """Every unit of the TTT-MLP 125M workload (b = 16); the oracle backward
    runs one unit per call on a thread pool (it keeps all T + 1 states)."""
    x = inputs.make_inputs(4)
    rng = np.random.default_rng(820)
    dz = (rng.standard_normal(x.q.shape) * 0.1).astype(np.float32)
    _, _, got = run_fwd_bwd(x, 16, dz)
    assert all(np.isfinite(a).all() for a in got)
    dzu = dz.reshape(-1, x.wl.T, 64)

    def one(u):
        s = x.units([u])
        return oracle.mlp_bwd(s.q, s.k, s.v, s.eta, s.w1, s.w2, 16, dzu[u][None, None])

    per = gu.oracle_units_parallel(one, x.wl.units)
    ref = [np.concatenate([p[i] for p in per], axis=1).reshape(got[i].shape) for i in range(6)]
    print("MLP 125M backward:", check(got, ref, "125M"))


@pytest.mark.parametrize("dtype, b", [("f32", 16), ("bf16", 16), ("bf16", 4), ("bf16", 1),
                                      ("bf16", 32)])
def test_forward_with_checkpoints_matches_plain_forward(dtype, b):
    """ttt_mlp_fwd and ttt_mlp_fwd_ckpt run the same kernel (the checkpoint
    variant only adds stores), so z and the final states are bit-identical."""
    x = case(1, 3, 70, dtype, seed=830)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    a = ttt_mlp_fwd(q, k, v, gu.f32(x.eta), gu.f32(x.w1), gu.f32(x.w2), b)
    c = ttt_mlp_fwd_ckpt(q, k, v, gu.f32(x.eta), gu.f32(x.w1), gu.f32(x.w2), b)
    torch.cuda.synchronize()
    for u, w in zip(a, c[:3]):
        assert torch.equal(u, w)


def test_backward_empty_sequence_and_rejected_arguments():
    x = case(1, 2, 16, "bf16", seed=840)
    e = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    ck1 = torch.empty(1, 2, 0, 256, 64, device="cuda")
    ck2 = torch.empty(1, 2, 0, 64, 256, device="cuda")
    d1 = torch.randn(1, 2, 256, 64, device="cuda")
    d2 = torch.randn(1, 2, 64, 256, device="cuda")
    g = ttt_mlp_bwd(e, e, e, torch.empty(1, 2, 0, device="cuda"), ck1, ck2, 16,
                    torch.empty(1, 2, 0, 64, device="cuda"), d1, d2)
    torch.cuda.synchronize()
    assert torch.equal(g[4], d1) and torch.equal(g[5], d2)  # no tokens: dW0 = dW_T
    q, k, v = (gu.dev(x, n) for n in "qkv")
    _, _, _, c1, c2 = ttt_mlp_fwd_ckpt(q, k, v, gu.f32(x.eta), gu.f32(x.w1), gu.f32(x.w2), 16)
    dz = torch.randn(1, 2, 16, 64, device="cuda")
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_mlp_bwd(q, k, v, gu.f32(x.eta), c1, c2, 24, dz)
