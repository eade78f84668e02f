"""TTT-MLP: HIP path (through the C ABI) against the fp64 primal oracle."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from test_rnn_layers_head_amd import TTTError, inputs, ttt_mlp_fwd

pytestmark = pytest.mark.gpu


def small(B, H, T, seed):
    return inputs.make_inputs(inputs.Workload("small-mlp", "mlp", B=B, H=H, T=T, hidden=256,
                                              seed=seed))


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("T", [1, 15, 16, 37, 100])
def test_small_parity(b, T):
    x = small(2, 2, T, seed=200 + T + b)
    z, w1, w2 = gu.run_mlp(x, b)
    zr, w1r, w2r = gu.oracle_mlp(x, b)
    print(f"T={T} b={b} z:", gu.assert_close(z, zr, "bf16", "z"),
          "w1:", gu.assert_close(w1, w1r, "bf16", "w1"), "w2:", gu.assert_close(w2, w2r, "bf16", "w2"))


def test_125m_workload_all_units():
    x = inputs.make_inputs(4)
    z, w1, w2 = gu.run_mlp(x, 16)
    assert np.isfinite(z).all()
    zr, w1r, w2r = gu.oracle_mlp(x, 16)
    print("MLP 125M z:", gu.assert_close_all_units(z, zr, "bf16", "z"),
          "w1:", gu.assert_close_all_units(w1, w1r, "bf16", "w1"),
          "w2:", gu.assert_close_all_units(w2, w2r, "bf16", "w2"))


def test_deterministic_reruns():
    x = small(2, 3, 70, seed=9)
    a = gu.run_mlp(x, 16)
    b = gu.run_mlp(x, 16)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_state_passing_in_place():
    x = small(1, 2, 96, seed=10)
    z, w1, w2 = gu.run_mlp(x, 16)
    T1 = 48
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta = gu.f32(x.eta)
    s1 = gu.f32(np.broadcast_to(x.w1, (1, 2, 256, 64)))
    s2 = gu.f32(np.broadcast_to(x.w2, (1, 2, 64, 256)))
    sl = lambda t, a, b_: t[:, :, a:b_].contiguous()
    za, _, _ = ttt_mlp_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(eta, 0, T1), s1, s2, 16,
                           w1_out=s1, w2_out=s2)
    zb, _, _ = ttt_mlp_fwd(sl(q, T1, 96), sl(k, T1, 96), sl(v, T1, 96), sl(eta, T1, 96), s1, s2, 16,
                           w1_out=s1, w2_out=s2)
    torch.cuda.synchronize()
    zz = torch.cat([za, zb], dim=2).cpu().numpy()
    assert gu.metrics(zz, z)["rel_l2"] < 1e-4
    assert gu.metrics(s1.cpu().numpy(), w1)["rel_l2"] < 1e-4
    assert gu.metrics(s2.cpu().numpy(), w2)["rel_l2"] < 1e-4


def test_empty_sequence_copies_state():
    x = small(2, 2, 0, seed=11)
    z, w1, w2 = gu.run_mlp(x, 16)
    assert z.shape == (2, 2, 0, 64)
    assert np.array_equal(w1, np.broadcast_to(x.w1, w1.shape))
    assert np.array_equal(w2, np.broadcast_to(x.w2, w2.shape))


def small_f32(B, H, T, seed):
    return inputs.make_inputs(inputs.Workload("small-mlp-f32", "mlp", B=B, H=H, T=T, hidden=256,
                                              qkv_dtype="f32", seed=seed))


@pytest.mark.parametrize("b", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 37, 130])
def test_fp32_inputs_parity(b, T):
    """fp32 q/k/v (the primal kernel, exact fp32 products): rel-L2 <= 1e-5."""
    x = small_f32(2, 2, T, seed=260 + T + b)
    z, w1, w2 = gu.run_mlp(x, b)
    zr, w1r, w2r = gu.oracle_mlp(x, b)
    print(f"fp32 T={T} b={b} z:", gu.assert_close(z, zr, "f32", "z"),
          "w1:", gu.assert_close(w1, w1r, "f32", "w1"), "w2:", gu.assert_close(w2, w2r, "f32", "w2"))


@pytest.mark.parametrize("b", [32, 48, 64])
@pytest.mark.parametrize("T", [16, 100, 200])
def test_long_minibatch_parity(b, T):
    """b a multiple of 16 above 16: the gradient point is held across tiles."""
    x = small(2, 2, T, seed=280 + T + b)
    z, w1, w2 = gu.run_mlp(x, b)
    zr, w1r, w2r = gu.oracle_mlp(x, b)
    print(f"T={T} b={b} z:", gu.assert_close(z, zr, "bf16", "z"),
          "w1:", gu.assert_close(w1, w1r, "bf16", "w1"), "w2:", gu.assert_close(w2, w2r, "bf16", "w2"))


def test_125m_workload_b64_all_units():
    x = inputs.make_inputs(4)
    z, w1, w2 = gu.run_mlp(x, 64)
    assert np.isfinite(z).all()
    zr, w1r, w2r = gu.oracle_mlp(x, 64)
    print("MLP 125M b=64 z:", gu.assert_close_all_units(z, zr, "bf16", "z"),
          "w1:", gu.assert_close_all_units(w1, w1r, "bf16", "w1"),
          "w2:", gu.assert_close_all_units(w2, w2r, "bf16", "w2"))


def test_unsupported_configurations_are_rejected():
    x = small(1, 1, 16, seed=12)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta, w1, w2 = gu.f32(x.eta), gu.f32(x.w1), gu.f32(x.w2)
    for b in (3, 24):  # neither b | 16 nor 16 | b
        with pytest.raises(TTTError) as e:
            ttt_mlp_fwd(q, k, v, eta, w1, w2, b)
        assert e.value.status == 4
