"""Backward of the TTT-Linear scan: HIP path (ttt_linear_fwd_ckpt +
ttt_linear_bwd through the C ABI) against the fp64 backward oracle.

Tolerance: the checkpointed states come from the bf16-input forward (its
hi/lo operand splits, ~2^-16 relative) and the backward's products use the
same hi/lo splits of every fp32 operand.  The bound is the bf16-input one of
the forward, rel-L2 <= 2e-3 and max|diff| / RMS <= 1e-2, on every gradient.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import oracle
from test_rnn_layers_head_amd import (TTTError, inputs, ttt_linear_bwd, ttt_linear_fwd,
                                      ttt_linear_fwd_ckpt)

pytestmark = pytest.mark.gpu


def run_fwd_bwd(x, dz, dwT=None):
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    z, w, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    grads = ttt_linear_bwd(q, k, v, eta, ck, 16, gu.f32(dz), None if dwT is None else gu.f32(dwT))
    torch.cuda.synchronize()
    return z, w, ck, [t.cpu().numpy() for t in grads]


def check(got, ref, what):
    for name, a, b in zip(("dq", "dk", "dv", "deta", "dw0"), got, ref):
        gu.assert_close(a, b, "bf16", f"{what} {name}")


@pytest.mark.parametrize("T", [1, 16, 37, 130])
def test_checkpoints_are_the_states_before_each_minibatch(T):
    x = inputs.make_inputs(inputs.Workload("ck", "linear", B=2, H=3, T=T, seed=700 + T))
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    z, w, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    z0, w00 = ttt_linear_fwd(q, k, v, eta, w0, 16)
    torch.cuda.synchronize()
    assert torch.equal(z, z0) and torch.equal(w, w00)  # same kernel arithmetic
    ck = ck.cpu().numpy()
    for m in range(ck.shape[2]):
        if m == 0:
            ref = np.broadcast_to(x.w0[None], ck[:, :, 0].shape)
        else:
            sub = inputs.Inputs(x.wl, x.q[:, :, :16 * m], x.k[:, :, :16 * m], x.v[:, :, :16 * m],
                                x.eta[:, :, :16 * m], x.w0)
            _, ref = oracle.linear(sub.q, sub.k, sub.v, sub.eta, sub.w0, 16)
        gu.assert_close(ck[:, :, m], ref, "bf16", f"checkpoint {m}")


@pytest.mark.parametrize("T", [16, 37, 130])
@pytest.mark.parametrize("with_dwT", [False, True])
def test_backward_parity(T, with_dwT):
    x = inputs.make_inputs(inputs.Workload("bwd", "linear", B=2, H=3, T=T, seed=710 + T))
    rng = np.random.default_rng(711 + T)
    dz = rng.standard_normal(x.q.shape).astype(np.float32)
    dwT = rng.standard_normal((2, 3, 64, 64)).astype(np.float32) if with_dwT else None
    _, _, _, got = run_fwd_bwd(x, dz, dwT)
    ref = oracle.linear_bwd(x.q, x.k, x.v, x.eta, x.w0, 16, dz, dwT)
    check(got, ref, f"T={T}")


def test_backward_per_unit_initial_state_and_eta_zero_tokens():
    x = inputs.make_inputs(inputs.Workload("bwd2", "linear", B=2, H=2, T=50, seed=720))
    rng = np.random.default_rng(721)
    x.w0 = (rng.standard_normal((2, 2, 64, 64)) * 0.02).astype(np.float32)
    x.eta[:, :, 5:9] = 0.0
    dz = rng.standard_normal(x.q.shape).astype(np.float32)
    _, _, _, got = run_fwd_bwd(x, dz)
    ref = oracle.linear_bwd(x.q, x.k, x.v, x.eta, x.w0, 16, dz)
    check(got, ref, "per-unit w0")


def test_backward_1p3b_workload_all_units():
    """Every unit of the 1.3B workload: the oracle backward runs one unit per
    call on a thread pool (it keeps all T states of a unit, 268 MB each)."""
    x = inputs.make_inputs(3)
    rng = np.random.default_rng(730)
    dz = (rng.standard_normal(x.q.shape) * 0.1).astype(np.float32)
    _, _, _, got = run_fwd_bwd(x, dz)
    assert all(np.isfinite(a).all() for a in got)
    dzu = dz.reshape(-1, x.wl.T, 64)

    def one(u):
        s = x.units([u])
        return oracle.linear_bwd(s.q, s.k, s.v, s.eta, s.w0, 16, dzu[u][None, None])

    per = gu.oracle_units_parallel(one, x.wl.units)
    ref = [np.concatenate([p[i] for p in per], axis=1).reshape(got[i].shape) for i in range(5)]
    check(got, ref, "1.3B")


def test_backward_empty_sequence_and_rejected_arguments():
    x = inputs.make_inputs(inputs.Workload("bwd0", "linear", B=1, H=2, T=16, seed=740))
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    dwT = torch.randn(1, 2, 64, 64, device="cuda")
    e = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    ck0 = torch.empty(1, 2, 0, 64, 64, device="cuda")
    grads = ttt_linear_bwd(e, e, e, torch.empty(1, 2, 0, device="cuda"), ck0, 16,
                           torch.empty(1, 2, 0, 64, device="cuda"), dwT)
    torch.cuda.synchronize()
    assert torch.equal(grads[4], dwT)  # no tokens: dL/dW0 = dL/dW_T
    _, _, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    dz = torch.randn(1, 2, 16, 64, device="cuda")
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_linear_bwd(q, k, v, eta, ck, 24, dz)
    ck4 = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 4)[2]
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):  # chunks need bf16, b = 16
        ttt_linear_bwd(q, k, v, eta, ck4, 4, dz, seq_chunks=2)


# ------------------------------------------------ any b, fp32 inputs
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 16, 32, 48, 64])
@pytest.mark.parametrize("T", [1, 37, 120, 130])
def test_any_minibatch_checkpoints_and_backward(dtype, b, T):
    """bf16 with b < 16: the b = 16 dual-form kernels with one mini-batch per
    zero-padded tile; bf16 with b > 16: the dual-form backward with the
    gradient point held across b / 16 tiles (T = 120 ends in a mini-batch of
    several tiles, T = 130 in one of a single ragged tile); fp32 q/k/v: the
    primal-form kernels.
    Checkpoints (one per mini-batch) against the oracle's states, then every
    gradient against the oracle backward, with dW_T given."""
    if dtype == "bf16" and b == 16:
        pytest.skip("the dual-form kernels, tested above")
    x = inputs.make_inputs(inputs.Workload("bwdb", "linear", B=2, H=2, T=T, qkv_dtype=dtype,
                                           seed=760 + T + b))
    rng = np.random.default_rng(761 + T + b)
    dz = rng.standard_normal(x.q.shape).astype(np.float32)
    dwT = rng.standard_normal((2, 2, 64, 64)).astype(np.float32)
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    z, w, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, b)
    grads = ttt_linear_bwd(q, k, v, eta, ck, b, gu.f32(dz), gu.f32(dwT))
    torch.cuda.synchronize()
    zr, wr = oracle.linear(x.q, x.k, x.v, x.eta, x.w0, b)
    gu.assert_close(z.cpu().numpy(), zr, dtype, "z")
    gu.assert_close(w.cpu().numpy(), wr, dtype, "w_T")
    ck = ck.cpu().numpy()
    assert ck.shape[2] == (T + b - 1) // b
    for m in range(1, ck.shape[2]):
        _, ref = oracle.linear(x.q[:, :, :b * m], x.k[:, :, :b * m], x.v[:, :, :b * m],
                               x.eta[:, :, :b * m], x.w0, b)
        gu.assert_close(ck[:, :, m], ref, dtype, f"checkpoint {m}")
    ref = oracle.linear_bwd(x.q, x.k, x.v, x.eta, x.w0, b, dz, dwT)
    got = [t.cpu().numpy() for t in grads]
    for name, a, r in zip(("dq", "dk", "dv", "deta", "dw0"), got, ref):
        m_ = gu.assert_close(a, r, dtype, f"T={T} b={b} {name}")
    print(f"{dtype} T={T} b={b} last:", m_)


@pytest.mark.parametrize("b", [1, 4, 64])
def test_backward_1p3b_workload_any_minibatch_sampled_units(b):
    """The 1.3B workload with b in {1, 4} (the dual-form kernels on padded
    tiles) and 64 (the dual form with the gradient point held across four
    tiles): 16 units spread over the batch and heads against the oracle
    backward."""
    x = inputs.make_inputs(3)
    rng = np.random.default_rng(770 + b)
    dz = (rng.standard_normal(x.q.shape) * 0.1).astype(np.float32)
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    _, _, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, b)
    got = [t.cpu().numpy() for t in ttt_linear_bwd(q, k, v, eta, ck, b, gu.f32(dz))]
    torch.cuda.synchronize()
    idx = list(range(0, 128, 8))
    dzu = dz.reshape(-1, x.wl.T, 64)

    def one(u):
        s_ = x.units([u])
        return oracle.linear_bwd(s_.q, s_.k, s_.v, s_.eta, s_.w0, b, dzu[u][None, None])

    per = gu.oracle_units_parallel(lambda i: one(idx[i]), len(idx))
    for i, name in enumerate(("dq", "dk", "dv", "deta", "dw0")):
        ref = np.concatenate([p[i] for p in per], axis=1)
        sub = got[i].reshape(-1, *got[i].shape[2:])[idx][None]
        gu.assert_close(sub, ref, "bf16", f"1.3B b={b} {name}")


# ---------------------------------------------------------------- sequence chunks
@pytest.mark.parametrize("T,P", [(768, 2), (768, 4), (576, 3)])
@pytest.mark.parametrize("with_dwT", [False, True])
def test_chunked_backward_parity(T, P, with_dwT):
    """P chunks of T / P tokens (192 and 384: 12 and 24 tiles per chunk)."""
    x = inputs.make_inputs(inputs.Workload("bwdc", "linear", B=1, H=2, T=T, seed=750 + P))
    rng = np.random.default_rng(751 + T + P)
    dz = rng.standard_normal(x.q.shape).astype(np.float32)
    dwT = rng.standard_normal((1, 2, 64, 64)).astype(np.float32) if with_dwT else None
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    _, _, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    dwT_d = None if dwT is None else gu.f32(dwT)
    got = ttt_linear_bwd(q, k, v, eta, ck, 16, gu.f32(dz), dwT_d, seq_chunks=P)
    one = ttt_linear_bwd(q, k, v, eta, ck, 16, gu.f32(dz), dwT_d, seq_chunks=1)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in got]
    ref = oracle.linear_bwd(x.q, x.k, x.v, x.eta, x.w0, 16, dz, dwT)
    check(got, ref, f"T={T} P={P}")
    check(got, [t.cpu().numpy() for t in one], f"T={T} P={P} vs one pass")


def test_chunked_backward_is_deterministic_and_ignores_prior_output_contents():
    """dq's memory serves the chunk maps first: NaN there beforehand changes nothing."""
    x = inputs.make_inputs(inputs.Workload("bwdd", "linear", B=1, H=2, T=768, seed=760))
    dz = gu.f32(np.random.default_rng(761).standard_normal(x.q.shape).astype(np.float32))
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    _, _, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    a = ttt_linear_bwd(q, k, v, eta, ck, 16, dz, seq_chunks=4)
    outs = [torch.full_like(t, float("nan")) for t in a]
    from test_rnn_layers_head_amd import _lib
    from test_rnn_layers_head_amd.api import _ptr
    _lib.check(_lib.lib().ttt_linear_bwd_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(ck), 1, 2, 768, 64, 16, _lib.TTT_BF16, _ptr(dz),
        None, *(_ptr(t) for t in outs), torch.cuda.current_stream().cuda_stream, 4))
    torch.cuda.synchronize()
    assert all(torch.equal(u, w) for u, w in zip(a, outs))


def test_long_sequence_checkpoints_and_backward_in_chunks():
    """1 x 2 x 8192: the checkpointing forward and the backward both take 8
    chunks (units * P <= 256, chunks of 1024 tokens); sampled checkpoints and
    every gradient against the oracle."""
    from test_rnn_layers_head_amd import ttt_linear_fwd_plan
    assert ttt_linear_fwd_plan(1, 2, 8192, 16)[1] == 8
    x = inputs.make_inputs(inputs.Workload("bwdl", "linear", B=1, H=2, T=8192, seed=770))
    rng = np.random.default_rng(771)
    dz = (rng.standard_normal(x.q.shape) * 0.1).astype(np.float32)
    z, w, ck, got = run_fwd_bwd(x, dz)
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    z1, w1 = ttt_linear_fwd(q, k, v, gu.f32(x.eta), gu.f32(x.w0), 16)
    torch.cuda.synchronize()
    assert torch.equal(z, z1) and torch.equal(w, w1)  # same chunked passes, plus the checkpoints
    ck = ck.cpu().numpy()
    for m in (1, 64, 65, 300, 511):  # inside chunks and at chunk starts (every 64 tiles)
        _, ref = oracle.linear(x.q[:, :, :16 * m], x.k[:, :, :16 * m], x.v[:, :, :16 * m],
                               x.eta[:, :, :16 * m], x.w0, 16)
        gu.assert_close(ck[:, :, m], ref, "bf16", f"checkpoint {m}")
    ref = oracle.linear_bwd(x.q, x.k, x.v, x.eta, x.w0, 16, dz)
    check(got, ref, "T=8192 chunked")


def test_chunked_backward_rejects():
    x = inputs.make_inputs(inputs.Workload("bwdr", "linear", B=1, H=1, T=768, seed=780))
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    _, _, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    dz = torch.zeros(1, 1, 768, 64, device="cuda")
    for P in (-1, 5, 8):  # negative; T % P != 0; T / P < 192
        with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
            ttt_linear_bwd(q, k, v, eta, ck, 16, dz, seq_chunks=P)


def test_chunked_backward_graph_replays_match_eager():
    """The chunked backward's four launches captured in one HIP graph: every
    replay gives exactly the eager result (outputs NaN-filled before each)."""
    x = inputs.make_inputs(inputs.Workload("bwdg", "linear", B=1, H=2, T=1536, seed=790))
    q, k, v = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    dz = gu.f32(np.random.default_rng(791).standard_normal(x.q.shape).astype(np.float32))
    dwT = gu.f32(np.random.default_rng(792).standard_normal((1, 2, 64, 64)).astype(np.float32))
    _, _, ck = ttt_linear_fwd_ckpt(q, k, v, eta, w0, 16)
    ref = ttt_linear_bwd(q, k, v, eta, ck, 16, dz, dwT, seq_chunks=4)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            outs = ttt_linear_bwd(q, k, v, eta, ck, 16, dz, dwT, stream=s, seq_chunks=4)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), rep
        assert torch.isfinite(scratch)
