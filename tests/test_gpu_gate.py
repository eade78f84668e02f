"""GPU parity of the inner learning-rate gate ("论文速览 | TTT", §4.6),
eta = eta_base * sigmoid(theta_lr[h] . x[b, t]), of its backward, and of the
gated scans, against the fp64 oracle.

Tolerance of the gate, from its arithmetic: each product theta_i x_i is
exact on the device except for theta's three-term bf16 split, which drops at
most 2^-27 |theta_i| per element; the n = dx products are summed in fp32 in
some order, within n 2^-24 sum|theta_i x_i| of the exact sum.  The logit
error therefore stays below E = (n + 1) 2^-24 S with S = sum |theta_i x_i|,
and sigmoid' <= 1/4 turns that into |d eta| <= |eta_base| (E / 4) plus a few
ulp of the fp32 sigmoid (8 ulp of eta_base allowed).  The gated scans then
meet the scan bounds (rel-L2 <= 2e-3 and max/RMS <= 1e-2 for bf16 q/k/v).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import oracle
from test_rnn_layers_head_amd import (TTTError, inputs, ttt_linear_gated_fwd, ttt_lr_gate,
                                      ttt_lr_gate_bwd, ttt_mlp_gated_fwd)

pytestmark = pytest.mark.gpu


def bf16_dev(raw):
    return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).cuda().view(torch.bfloat16)


def draw_gate(seed, B, T, H, dx, theta_scale=None):
    rng = np.random.default_rng(seed)
    raw = inputs.bf16_bits(rng.standard_normal((B, T, dx)))
    x = inputs.bf16_to_f32(raw)
    s = 1.0 / np.sqrt(dx) if theta_scale is None else theta_scale
    theta = (rng.standard_normal((H, dx)) * s).astype(np.float32)
    return raw, x, theta


def gate_bound(x, theta, eta_base):
    """Per-element bound on |eta_gpu - eta_exact| (module docstring)."""
    dx = x.shape[-1]
    S = np.einsum("btd,hd->bht", np.abs(x.astype(np.float64)), np.abs(theta.astype(np.float64)))
    E = (dx + 1) * 2.0 ** -24 * S
    return abs(eta_base) * (E / 4 + 8 * 2.0 ** -24)


def check_gate(got, x, theta, eta_base):
    ref = oracle.lr_gate(x, theta, eta_base)
    err = np.abs(got.astype(np.float64) - ref)
    bound = gate_bound(x, theta, eta_base)
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"gate error {err.max():.3e} exceeds its bound (ratio {worst:.2f})"
    return ref


@pytest.mark.parametrize("B,T,H,dx", [
    (2, 100, 5, 96),     # ragged token tail, one partial head block, fewer steps than waves
    (1, 37, 16, 32),     # a single 32-wide step
    (3, 64, 40, 256),    # two head passes (32 + 8)
    (1, 300, 33, 2048),  # the 1.3B layer width, a head block of one
])
@pytest.mark.parametrize("tpw", [32, 64])
def test_gate_parity(B, T, H, dx, tpw):
    raw, x, theta = draw_gate(100 + B * T + H + dx, B, T, H, dx)
    eta = ttt_lr_gate(bf16_dev(raw), gu.f32(theta), 0.1, tokens_per_workgroup=tpw)
    torch.cuda.synchronize()
    check_gate(eta.cpu().numpy(), x, theta, 0.1)


def test_gate_launch_shapes_agree_bit_for_bit():
    raw, x, theta = draw_gate(7, 2, 200, 12, 768)
    xd, td = bf16_dev(raw), gu.f32(theta)
    a = ttt_lr_gate(xd, td, 1.0, tokens_per_workgroup=32)
    b = ttt_lr_gate(xd, td, 1.0, tokens_per_workgroup=64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gate_saturation_sign_and_zero_vector():
    # large logits saturate to eta_base and 0; theta = 0 gives eta_base / 2
    B, T, H, dx = 1, 40, 3, 64
    raw, x, theta = draw_gate(11, B, T, H, dx, theta_scale=4.0)
    eta = ttt_lr_gate(bf16_dev(raw), gu.f32(theta), -0.5).cpu().numpy()
    check_gate(eta, x, theta, -0.5)
    assert np.all(eta <= 0) and np.all(eta >= -0.5)
    z = ttt_lr_gate(bf16_dev(raw), torch.zeros(H, dx, device="cuda"), 2.0)
    torch.cuda.synchronize()
    assert torch.all(z == 1.0)


def test_gate_1p3b_width_full_workload():
    # the gate of the gated 1.3B workload in full (32768 tokens x 32 heads x 2048)
    x = inputs.make_inputs(inputs.workload(8))
    eta = ttt_lr_gate(bf16_dev(x.gate_x_raw), gu.f32(x.theta_lr), x.eta_base)
    torch.cuda.synchronize()
    got = eta.cpu().numpy()
    # sampled (batch, head) rows against the oracle, all tokens of each
    rng = np.random.default_rng(0)
    for bi, h in zip(rng.integers(0, x.wl.B, 6), rng.integers(0, x.wl.H, 6)):
        check_gate(got[bi:bi + 1, h:h + 1], x.gate_x[bi:bi + 1], x.theta_lr[h:h + 1], x.eta_base)
    # the logits are ~N(0, 1): eta spreads over (0, eta_base)
    assert 0.3 * x.eta_base < got.mean() < 0.7 * x.eta_base


@pytest.mark.parametrize("wid", [9])
def test_linear_gated_workload(wid):
    x = inputs.make_inputs(inputs.workload(wid))
    z, w, eta = ttt_linear_gated_fwd(gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"),
                                     bf16_dev(x.gate_x_raw), gu.f32(x.theta_lr), x.eta_base,
                                     gu.f32(x.w0), 16)
    torch.cuda.synchronize()
    eta_ref = check_gate(eta.cpu().numpy(), x.gate_x, x.theta_lr, x.eta_base)
    zr, wr = oracle.linear(x.q, x.k, x.v, eta_ref, x.w0, 16)
    gu.assert_close(z.cpu().numpy(), zr, "bf16", "z")
    gu.assert_close(w.cpu().numpy(), wr, "bf16", "w")


@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_linear_gated_small(b):
    B, H, T, d, dx = 2, 3, 100, 64, 192
    x = inputs.make_inputs(inputs.Workload("gated-small", "linear", B=B, H=H, T=T, seed=21,
                                           gate_dx=dx))
    z, w, eta = ttt_linear_gated_fwd(gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"),
                                     bf16_dev(x.gate_x_raw), gu.f32(x.theta_lr), 1.0,
                                     gu.f32(x.w0), b)
    torch.cuda.synchronize()
    eta_ref = check_gate(eta.cpu().numpy(), x.gate_x, x.theta_lr, 1.0)
    zr, wr = oracle.linear(x.q, x.k, x.v, eta_ref, x.w0, b)
    gu.assert_close(z.cpu().numpy(), zr, "bf16", "z")
    gu.assert_close(w.cpu().numpy(), wr, "bf16", "w")


def test_linear_gated_1p3b_sampled_units():
    x = inputs.make_inputs(inputs.workload(8))
    z, w, eta = ttt_linear_gated_fwd(gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"),
                                     bf16_dev(x.gate_x_raw), gu.f32(x.theta_lr), x.eta_base,
                                     gu.f32(x.w0), 16)
    torch.cuda.synchronize()
    z, w = z.cpu().numpy(), w.cpu().numpy()
    idx = np.array([0, 45, 77, 127])
    sub = x.units(idx)
    bi, h = idx // x.wl.H, idx % x.wl.H
    eta_ref = np.stack([oracle.lr_gate(x.gate_x[b:b + 1], x.theta_lr[hh:hh + 1], x.eta_base)[0, 0]
                        for b, hh in zip(bi, h)])[None]
    zr, wr = oracle.linear(sub.q, sub.k, sub.v, eta_ref, sub.w0[:, :], 16)
    gu.assert_close(z.reshape(-1, *z.shape[2:])[idx][None], zr, "bf16", "z")
    gu.assert_close(w.reshape(-1, *w.shape[2:])[idx][None], wr, "bf16", "w")


def test_mlp_gated_small():
    B, H, T, dx = 1, 2, 48, 128
    x = inputs.make_inputs(inputs.Workload("gated-mlp", "mlp", B=B, H=H, T=T, hidden=256, seed=22,
                                           gate_dx=dx))
    z, w1, w2, eta = ttt_mlp_gated_fwd(gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"),
                                       bf16_dev(x.gate_x_raw), gu.f32(x.theta_lr), 0.1,
                                       gu.f32(x.w1), gu.f32(x.w2), 16)
    torch.cuda.synchronize()
    eta_ref = check_gate(eta.cpu().numpy(), x.gate_x, x.theta_lr, 0.1)
    zr, w1r, w2r = oracle.mlp(x.q, x.k, x.v, eta_ref, x.w1, x.w2, 16)
    gu.assert_close(z.cpu().numpy(), zr, "bf16", "z")
    gu.assert_close(w1.cpu().numpy(), w1r, "bf16", "w1")
    gu.assert_close(w2.cpu().numpy(), w2r, "bf16", "w2")


def test_gated_empty_sequence_and_rejected_arguments():
    x = inputs.make_inputs(inputs.Workload("gated-empty", "linear", B=1, H=2, T=0, seed=23,
                                           gate_dx=64))
    z, w, eta = ttt_linear_gated_fwd(gu.dev(x, "q"), gu.dev(x, "k"), gu.dev(x, "v"),
                                     bf16_dev(x.gate_x_raw), gu.f32(x.theta_lr), 1.0,
                                     gu.f32(x.w0), 16)
    torch.cuda.synchronize()
    assert z.numel() == 0 and eta.numel() == 0
    np.testing.assert_array_equal(w.cpu().numpy(), np.broadcast_to(x.w0, w.shape))
    raw, _, theta = draw_gate(3, 1, 16, 2, 48)
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_lr_gate(bf16_dev(raw), gu.f32(theta), 1.0)


# Backward of the gate.  dtheta_lr sums products of exact bf16 x with da as
# hi + lo bf16 (~2^-17 relative each) in fp32 over the tokens; dx sums fp32
# products over the heads; da comes from the forward's fp32 eta rather than
# the fp64 logit.  The bound is rel-L2 <= 2e-5 on both.
TOL_GATE_BWD = 2e-5


def check_gate_bwd(B, T, H, dx, eta_base, seed):
    raw, x, theta = draw_gate(seed, B, T, H, dx)
    deta = np.random.default_rng(seed + 1).standard_normal((B, H, T)).astype(np.float32)
    xd, td = bf16_dev(raw), gu.f32(theta)
    eta = ttt_lr_gate(xd, td, eta_base)
    dth, dxg = ttt_lr_gate_bwd(xd, td, eta_base, eta, gu.f32(deta))
    torch.cuda.synchronize()
    rth, rx = oracle.lr_gate_bwd(x, theta, eta_base, deta)
    m1, m2 = gu.metrics(dth.cpu().numpy(), rth), gu.metrics(dxg.cpu().numpy(), rx)
    assert m1["rel_l2"] <= TOL_GATE_BWD and m2["rel_l2"] <= TOL_GATE_BWD, (m1, m2)


@pytest.mark.parametrize("B,T,H,dx", [
    (2, 100, 5, 96),     # 32-column groups, ragged token chunks
    (1, 37, 16, 32),
    (3, 64, 40, 256),    # two passes of heads
    (1, 300, 33, 2048),
    (1, 5, 12, 64),      # fewer tokens than heads: one chunk, no scratch
    (9, 1, 2, 32),       # one-token sequences: every token starts a batch
    (6, 3, 3, 64),       # sequences shorter than a four-token group
    (2, 50, 36, 96),     # two head passes on 32-column tiles
    (2, 33, 20, 160),    # ragged sequences, one 32-head pass, 32-column tiles
])
def test_gate_bwd_parity(B, T, H, dx):
    check_gate_bwd(B, T, H, dx, 0.1, 200 + B + T + H + dx)


def test_gate_bwd_1p3b_width():
    # 8192 tokens of the 1.3B layer width: 16 token chunks
    check_gate_bwd(1, 8192, 32, 2048, 0.1, 300)


def test_gate_bwd_is_deterministic_and_handles_empty_dims():
    raw, x, theta = draw_gate(5, 2, 500, 12, 768)
    xd, td = bf16_dev(raw), gu.f32(theta)
    eta = ttt_lr_gate(xd, td, 1.0)
    deta = torch.randn(2, 12, 500, device="cuda")
    a1, b1 = ttt_lr_gate_bwd(xd, td, 1.0, eta, deta)
    a2, b2 = ttt_lr_gate_bwd(xd, td, 1.0, eta, deta)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(b1, b2)
    # no tokens: dtheta is zero
    e0 = torch.empty(1, 0, 64, dtype=torch.bfloat16, device="cuda")
    th = torch.randn(3, 64, device="cuda")
    z = torch.empty(1, 3, 0, device="cuda")
    dth0 = torch.full((3, 64), 7.0, device="cuda")
    dth, dxg = ttt_lr_gate_bwd(e0, th, 1.0, z, z, dtheta_lr=dth0)
    torch.cuda.synchronize()
    assert torch.all(dth == 0) and dxg.numel() == 0


def test_gate_and_backward_graph_replays_match_eager():
    """The gate and its backward captured in one HIP graph (the backward
    sizes its grids with host-side occupancy queries, which capture allows):
    every replay, with unrelated eager work between replays, gives exactly
    the eager results."""
    B, T, H, dx = 2, 256, 12, 768
    raw, x, theta = draw_gate(77, B, T, H, dx)
    deta = gu.f32(np.random.default_rng(78).standard_normal((B, H, T)).astype(np.float32))
    xd, td = bf16_dev(raw), gu.f32(theta)
    eta_e = ttt_lr_gate(xd, td, 0.1)
    dth_e, dx_e = ttt_lr_gate_bwd(xd, td, 0.1, eta_e, deta)
    torch.cuda.synchronize()
    eta = torch.empty_like(eta_e)
    dth, dxg = torch.empty_like(dth_e), torch.empty_like(dx_e)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ttt_lr_gate(xd, td, 0.1, eta=eta)
            ttt_lr_gate_bwd(xd, td, 0.1, eta, deta, dtheta_lr=dth, dx=dxg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        eta.fill_(float("nan"))
        dth.fill_(float("nan"))
        dxg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        assert torch.equal(eta, eta_e) and torch.equal(dth, dth_e) and torch.equal(dxg, dx_e), rep
        assert torch.isfinite(scratch)
