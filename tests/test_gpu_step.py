"""Decode steps (one token per unit, primal form): HIP path (through the C
ABI) against the fp64 step oracle, and whole sequences replayed step by step
against the fp64 scan oracles.

Tolerance.  A step is plain fp32 arithmetic (64-term dot products, the rank-1
update, for the LayerNorm variant three row reductions) on exact bf16 or
fp32 inputs, so one step agrees with fp64 to ~1e-7 relative; the bound is
the fp32 one, rel-L2 <= 1e-5, on z and both states.  Replayed sequences
accumulate the rounding of every step: rel-L2 <= 1e-5 for the bare model,
1e-4 for the LayerNorm one over 40 tokens.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from oracle import oracle
from test_rnn_layers_head_amd import TTTError, inputs, ttt_linear_ln_step, ttt_linear_step

pytestmark = pytest.mark.gpu


def close(got, ref, what, tol=1e-5):
    m = gu.metrics(got, ref)
    assert m["rel_l2"] <= tol, (what, m)
    return m


def token_inputs(B, H, dtype, seed):
    """One token's q, k, v, eta (host fp32 values and device tensors)."""
    wl = inputs.Workload("step", "linear", B=B, H=H, T=1, qkv_dtype=dtype, seed=seed)
    x = inputs.make_inputs(wl)
    host = {n: getattr(x, n)[:, :, 0] for n in ("q", "k", "v")}
    host["eta"] = x.eta[:, :, 0]
    dev = {}
    for n in ("q", "k", "v"):
        a = np.ascontiguousarray(getattr(x, n + "_raw")[:, :, 0])
        if a.dtype == np.uint16:
            dev[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            dev[n] = torch.from_numpy(a).cuda()
    dev["eta"] = gu.f32(host["eta"])
    return host, dev


def states(B, H, scale, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((B, H, 64, 64)) * scale).astype(np.float32)
    wg = (rng.standard_normal((B, H, 64, 64)) * scale).astype(np.float32)
    return w, wg


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 16])
def test_linear_step_parity(dtype, b):
    B, H = 3, 5
    host, dev = token_inputs(B, H, dtype, seed=500 + b)
    w, wg = states(B, H, 0.05, seed=501)
    pos = np.array([0, 5, 17], dtype=np.int32)
    wd, wgd = gu.f32(w), gu.f32(wg)
    z = ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], wd, wgd,
                        torch.from_numpy(pos).cuda(), b)
    torch.cuda.synchronize()
    zr, wr, wgr = oracle.linear_step(host["q"], host["k"], host["v"], host["eta"], w, wg, pos, b)
    close(z.cpu().numpy(), zr, "z")
    close(wd.cpu().numpy(), wr, "w")
    close(wgd.cpu().numpy(), wgr, "w_gp")


def test_linear_step_b1_without_gradient_point():
    B, H = 2, 4
    host, dev = token_inputs(B, H, "bf16", seed=510)
    w, _ = states(B, H, 0.05, seed=511)
    pos = np.array([3, 8], dtype=np.int32)
    wd = gu.f32(w)
    z = ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], wd, None,
                        torch.from_numpy(pos).cuda(), 1)
    torch.cuda.synchronize()
    zr, wr, _ = oracle.linear_step(host["q"], host["k"], host["v"], host["eta"], w, np.zeros_like(w),
                                   pos, 1)
    close(z.cpu().numpy(), zr, "z")
    close(wd.cpu().numpy(), wr, "w")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 3, 16])
def test_linear_ln_step_parity(dtype, b):
    B, H = 3, 5
    host, dev = token_inputs(B, H, dtype, seed=520 + b)
    w, wg = states(B, H, 0.125, seed=521)
    rng = np.random.default_rng(522)
    gamma = (1 + 0.2 * rng.standard_normal((H, 64))).astype(np.float32)
    beta = (0.1 * rng.standard_normal((H, 64))).astype(np.float32)
    pos = np.array([0, 7, 32], dtype=np.int32)
    wd, wgd = gu.f32(w), gu.f32(wg)
    z = ttt_linear_ln_step(dev["q"], dev["k"], dev["v"], dev["eta"], wd, wgd,
                           torch.from_numpy(pos).cuda(), gu.f32(gamma), gu.f32(beta), 1e-5, b)
    torch.cuda.synchronize()
    zr, wr, wgr = oracle.linear_ln_step(host["q"], host["k"], host["v"], host["eta"], w, wg, pos,
                                        gamma, beta, 1e-5, b)
    close(z.cpu().numpy(), zr, "z")
    close(wd.cpu().numpy(), wr, "w")
    close(wgd.cpu().numpy(), wgr, "w_gp")


def _replay(x, b, step, T):
    """Runs T decode steps over x's tokens; returns z [B, H, T, d]."""
    B, H = x.wl.B, x.wl.H
    qd, kd, vd = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta = gu.f32(x.eta)
    zs = []
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
        zs.append(step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                       vd[:, :, t].contiguous(), eta[:, :, t].contiguous(), pos).cpu().numpy())
    return np.stack(zs, axis=2)


@pytest.mark.parametrize("b", [4, 16])
def test_linear_steps_replay_the_scan(b):
    x = inputs.make_inputs(inputs.Workload("replay", "linear", B=2, H=3, T=40, seed=530 + b))
    w = gu.f32(np.broadcast_to(x.w0[None], (2, 3, 64, 64)))
    wg = torch.zeros_like(w)
    z = _replay(x, b, lambda q, k, v, e, p: ttt_linear_step(q, k, v, e, w, wg, p, b), 40)
    torch.cuda.synchronize()
    zr, wr = oracle.linear(x.q, x.k, x.v, x.eta, x.w0, b)
    close(z, zr, "z")
    close(w.cpu().numpy(), wr, "w_T")


@pytest.mark.parametrize("b", [1, 4, 16])
def test_linear_ln_steps_replay_the_scan(b):
    x = inputs.make_inputs(inputs.Workload("replay-ln", "linear_ln", B=2, H=3, T=40, seed=540 + b,
                                           eta_scale=0.02, w_scale=0.125))
    w = gu.f32(np.broadcast_to(x.w0[None], (2, 3, 64, 64)))
    wg = torch.zeros_like(w)
    g, be = gu.f32(x.ln_gamma), gu.f32(x.ln_beta)
    z = _replay(x, b, lambda q, k, v, e, p: ttt_linear_ln_step(q, k, v, e, w, wg, p, g, be,
                                                               x.wl.ln_eps, b), 40)
    torch.cuda.synchronize()
    zr, wr = oracle.linear_ln(x.q, x.k, x.v, x.eta, x.w0, x.ln_gamma, x.ln_beta, x.wl.ln_eps, b)
    close(z, zr, "z", 1e-4)
    close(w.cpu().numpy(), wr, "w_T", 1e-4)


def test_scan_then_steps_continue_a_sequence():
    # prefill 32 tokens with the scan (ends at a gradient point), decode 9 more
    x = inputs.make_inputs(inputs.Workload("resume", "linear", B=1, H=4, T=41, seed=550))
    from test_rnn_layers_head_amd import ttt_linear_fwd
    pre = 32
    qd, kd, vd = (gu.dev(x, n) for n in ("q", "k", "v"))
    eta = gu.f32(x.eta)
    _, w = ttt_linear_fwd(qd[:, :, :pre].contiguous(), kd[:, :, :pre].contiguous(),
                          vd[:, :, :pre].contiguous(), eta[:, :, :pre].contiguous(),
                          gu.f32(x.w0), 16)
    wg = torch.zeros_like(w)
    zs = []
    for t in range(pre, 41):
        pos = torch.full((1,), t, dtype=torch.int32, device="cuda")
        zs.append(ttt_linear_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                  vd[:, :, t].contiguous(), eta[:, :, t].contiguous(), w, wg, pos,
                                  16).cpu().numpy())
    torch.cuda.synchronize()
    zr, wr = oracle.linear(x.q, x.k, x.v, x.eta, x.w0, 16)
    close(np.stack(zs, axis=2), zr[:, :, pre:], "z", gu.TOL_BF16_REL)
    close(w.cpu().numpy(), wr, "w_T", gu.TOL_BF16_REL)


def test_step_rejected_arguments():
    host, dev = token_inputs(2, 2, "bf16", seed=560)
    w, wg = (gu.f32(a) for a in states(2, 2, 0.05, seed=561))
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(TTTError, match="TTT_ERR_NULL"):
        ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], w, None, pos, 16)
    with pytest.raises(TTTError, match="TTT_ERR_ALIAS"):
        ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], w, w, pos, 16)
    g = gu.f32(np.ones((2, 64)))
    with pytest.raises(TTTError, match="TTT_ERR_VALUE"):
        ttt_linear_ln_step(dev["q"], dev["k"], dev["v"], dev["eta"], w, wg, pos, g, g, 0.0, 16)
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], w, wg, pos, 0)


def mlp_states(B, H, seed, gp=True):
    rng = np.random.default_rng(seed)
    # W1 ~ N(0, 1) makes W1 k ~ N(0, 1) for |k| ~ 1, so GELU works away from 0
    mk = lambda shape, sc: (rng.standard_normal(shape) * sc).astype(np.float32)
    st = [mk((B, H, 256, 64), 1.0), mk((B, H, 64, 256), 1 / 16)]
    if gp:
        st += [mk((B, H, 256, 64), 1.0), mk((B, H, 64, 256), 1 / 16)]
    return st


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 4, 32])
def test_mlp_step_parity(dtype, b):
    from test_rnn_layers_head_amd import ttt_mlp_step
    B, H = 3, 2
    host, dev = token_inputs(B, H, dtype, seed=570 + b)
    w1, w2, w1g, w2g = mlp_states(B, H, seed=571)
    pos = np.array([0, 9, 32], dtype=np.int32)
    d = [gu.f32(a) for a in (w1, w2, w1g, w2g)]
    z = ttt_mlp_step(dev["q"], dev["k"], dev["v"], dev["eta"], *d, torch.from_numpy(pos).cuda(), b)
    torch.cuda.synchronize()
    ref = oracle.mlp_step(host["q"], host["k"], host["v"], host["eta"], w1, w2, w1g, w2g, pos, b)
    close(z.cpu().numpy(), ref[0], "z")
    for nm, got, want in zip(("w1", "w2", "w1_gp", "w2_gp"), d, ref[1:]):
        close(got.cpu().numpy(), want, nm)


def test_mlp_step_b1_without_gradient_points():
    from test_rnn_layers_head_amd import ttt_mlp_step
    B, H = 2, 2
    host, dev = token_inputs(B, H, "bf16", seed=580)
    w1, w2 = mlp_states(B, H, seed=581, gp=False)
    pos = np.array([4, 11], dtype=np.int32)
    d1, d2 = gu.f32(w1), gu.f32(w2)
    z = ttt_mlp_step(dev["q"], dev["k"], dev["v"], dev["eta"], d1, d2, None, None,
                     torch.from_numpy(pos).cuda(), 1)
    torch.cuda.synchronize()
    ref = oracle.mlp_step(host["q"], host["k"], host["v"], host["eta"], w1, w2, np.zeros_like(w1),
                          np.zeros_like(w2), pos, 1)
    close(z.cpu().numpy(), ref[0], "z")
    close(d1.cpu().numpy(), ref[1], "w1")
    close(d2.cpu().numpy(), ref[2], "w2")


@pytest.mark.parametrize("b", [4, 16])
def test_mlp_steps_replay_the_scan(b):
    from test_rnn_layers_head_amd import ttt_mlp_step
    x = inputs.make_inputs(inputs.Workload("replay-mlp", "mlp", B=2, H=2, T=24, hidden=256,
                                           seed=590 + b))
    w1 = gu.f32(np.broadcast_to(x.w1[None], (2, 2, 256, 64)))
    w2 = gu.f32(np.broadcast_to(x.w2[None], (2, 2, 64, 256)))
    w1g, w2g = torch.zeros_like(w1), torch.zeros_like(w2)
    z = _replay(x, b, lambda q, k, v, e, p: ttt_mlp_step(q, k, v, e, w1, w2, w1g, w2g, p, b), 24)
    torch.cuda.synchronize()
    zr, w1r, w2r = oracle.mlp(x.q, x.k, x.v, x.eta, x.w1, x.w2, b)
    close(z, zr, "z")
    close(w1.cpu().numpy(), w1r, "w1_T")
    close(w2.cpu().numpy(), w2r, "w2_T")


def test_graph_captured_steps_match_eager():
    # bench.py times the steps as a captured graph: every replay of the
    # captured step must give exactly what the same step gives eagerly
    # (eager work and synchronisations between the replays).
    B, H = 4, 8
    host, dev = token_inputs(B, H, "bf16", seed=600)
    w0, wg0 = states(B, H, 0.05, seed=601)
    pos_g = torch.tensor([0, 3, 16, 21], dtype=torch.int32, device="cuda")
    w, wg = gu.f32(w0), gu.f32(wg0)          # states advanced by the graph
    we, wge = gu.f32(w0), gu.f32(wg0)        # the same states advanced eagerly
    z = torch.empty(B, H, 64, device="cuda")
    ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], we.clone(), wge.clone(), pos_g, 16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], w, wg, pos_g, 16, z=z)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    w.copy_(gu.f32(w0))
    wg.copy_(gu.f32(wg0))
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        ze = ttt_linear_step(dev["q"], dev["k"], dev["v"], dev["eta"], we, wge, pos_g, 16)
        scratch = torch.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        assert torch.equal(z, ze), rep
        assert torch.equal(w, we) and torch.equal(wg, wge), rep
        assert torch.isfinite(scratch)
