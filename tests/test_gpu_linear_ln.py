"""TTT-Linear with the LayerNorm + residual inner model: HIP path (through the
C ABI) against the fp64 primal oracle.

Tolerance.  Q, K, V are exact bf16 values on both sides, so the difference
is the kernel's own arithmetic: fp32 state, sums and scalars, with every
product that feeds the recurrence taking its fp32 factors in three bf16
terms (~2^-24 relative, i.e. fp32 level) and the output products in two
(~2^-16).  The LayerNorm recurrence amplifies rounding along the sequence
(its loss ignores a common shift of W's rows and, up to eps, W's scale, and
rows with large gamma come to dominate a token's variance), so a plain fp32
evaluation of the same method, one token at a time, already differs from
the fp64 oracle by up to ~1e-3 of the RMS after 8k tokens.  Bounds:
  * up to 2k tokens: rel-L2 <= 1e-4 and max|diff| / RMS <= 1e-3;
  * the 8k-token workload: the bf16-input bound of the plain scan,
    rel-L2 <= 2e-3 and max|diff| / RMS <= 1e-2.
"""
import numpy as np
import pytest

import gpu_util as gu
from test_rnn_layers_head_amd import TTTError, inputs, ttt_linear_ln_fwd

pytestmark = pytest.mark.gpu

TOL_REL = 1e-4
TOL_MAX = 1e-3


def close(got, ref, what, rel=TOL_REL, mx=TOL_MAX):
    m = gu.metrics(got, ref)
    assert m["rel_l2"] <= rel and m["max_over_rms"] <= mx, (what, m)
    return m


def small(B, H, T, seed):
    wl = inputs.Workload("small-ln", "linear_ln", B=B, H=H, T=T, seed=seed, eta_scale=0.02,
                         w_scale=0.125)
    return inputs.make_inputs(wl)


@pytest.mark.parametrize("b", [16, 32, 48, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 37, 130])
def test_small_parity(b, T):
    x = small(2, 3, T, seed=300 + T + b)
    z, w = gu.run_linear_ln(x, b)
    zr, wr = gu.oracle_linear_ln(x, b)
    close(z, zr, "z")
    close(w, wr, "w_T")


def test_per_unit_initial_state_and_long_tail():
    x = small(2, 2, 16 * 9 + 5, seed=77)
    rng = np.random.default_rng(78)
    w0 = (rng.standard_normal((2, 2, 64, 64)) * 0.125).astype(np.float32)
    z, w = gu.run_linear_ln(x, 16, w0=w0)
    zr, wr = gu.oracle_linear_ln(x, 16, w0=w0)
    close(z, zr, "z")
    close(w, wr, "w_T")


def test_gamma_zero_keeps_state_and_outputs_q_plus_beta():
    # gamma = 0: the loss does not depend on W, the state never moves and
    # z = q + beta exactly.
    x = small(1, 2, 50, seed=79)
    gamma = np.zeros_like(x.ln_gamma)
    z, w = gu.run_linear_ln(x, 16, gamma=gamma)
    np.testing.assert_array_equal(w, np.broadcast_to(x.w0[None], w.shape))
    np.testing.assert_allclose(z, x.q + x.ln_beta[None, :, None, :], rtol=0, atol=1e-6)


@pytest.mark.parametrize("eps", [1e-8, 1e-2, 1.0])
def test_eps_range(eps):
    x = small(1, 2, 70, seed=80)
    z, w = gu.run_linear_ln(x, 16, eps=eps)
    zr, wr = gu.oracle_linear_ln(x, 16, eps=eps)
    close(z, zr, f"z eps={eps}")
    close(w, wr, f"w_T eps={eps}")


def test_zero_initial_state():
    # W0 = 0: every first-tile y is 0, its variance 0 and rs = 1/sqrt(eps).
    x = small(1, 1, 40, seed=81)
    w0 = np.zeros_like(x.w0)
    z, w = gu.run_linear_ln(x, 16, w0=w0, eps=1e-2)
    zr, wr = gu.oracle_linear_ln(x, 16, w0=w0, eps=1e-2)
    close(z, zr, "z")
    close(w, wr, "w_T")


def test_125m_ln_workload_full():
    x = inputs.make_inputs(7)
    z, w = gu.run_linear_ln(x, 16)
    zr, wr = gu.oracle_linear_ln(x, 16)
    print("LN 125M z:", close(z, zr, "z"), "w:", close(w, wr, "w"))


def test_1p3b_ln_workload_sampled_units():
    x = inputs.make_inputs(6)
    z, w = gu.run_linear_ln(x, 16)
    idx = [0, 37, 77, 127]
    sub = x.units(idx)
    zr, wr = gu.oracle_linear_ln(sub, 16)
    zs = z.reshape(-1, x.wl.T, 64)[idx][None]
    ws = w.reshape(-1, 64, 64)[idx][None]
    loose = dict(rel=gu.TOL_BF16_REL, mx=gu.TOL_BF16_MAX)
    print("LN 1.3B z:", close(zs, zr, "z", **loose), "w:", close(ws, wr, "w", **loose))
    assert np.isfinite(z).all() and np.isfinite(w).all()


def test_rejected_arguments():
    x = small(1, 1, 20, seed=82)
    with pytest.raises(TTTError, match="TTT_ERR_VALUE"):
        gu.run_linear_ln(x, 16, eps=0.0)
    with pytest.raises(TTTError, match="TTT_ERR_VALUE"):
        gu.run_linear_ln(x, 16, eps=float("nan"))
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        gu.run_linear_ln(x, 8)
    q = gu.f32(x.q)
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        ttt_linear_ln_fwd(q, gu.f32(x.k), gu.f32(x.v), gu.f32(x.eta), gu.f32(x.w0),
                          gu.f32(x.ln_gamma), gu.f32(x.ln_beta), 1e-5, 16)
