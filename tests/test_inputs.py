"""Seeded input generator: determinism, rounding, and the stated distributions."""
import numpy as np
import pytest
import torch

from test_rnn_layers_head_amd import inputs


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-3, 0.125, 1.0, 300.0)])
    # exact ties: low half exactly 0x8000 must round to even
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x.astype(np.float32), ties, -ties])
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_small_workload_is_deterministic_and_fp32():
    a = inputs.make_inputs(1)
    b = inputs.make_inputs(1)
    assert a.sha256() == b.sha256()
    assert a.q.dtype == np.float32 and a.q.shape == (1, 1, 256, 64)
    assert a.w0.shape == (1, 64, 64)
    assert 0.0 <= a.eta.min() and a.eta.max() <= 0.1


def test_bf16_workload_values_are_bf16_exact():
    wl = inputs.workload(2, B=2, H=3, T=64)
    x = inputs.make_inputs(wl)
    assert x.q_raw.dtype == np.uint16
    assert np.array_equal(inputs.bf16_bits(x.k), x.k_raw)
    assert abs(x.q.std() - 0.125) < 0.01
    assert 0.0 < x.eta.min() and x.eta.max() < 0.1
    assert abs(x.w0.std() - 0.02) < 0.002


def test_drift_workload_is_ar1():
    wl = inputs.workload(5, H=4, T=4096)
    x = inputs.make_inputs(wl)
    k = x.k.astype(np.float64)[0]
    lag1 = np.mean(k[:, 1:] * k[:, :-1]) / np.mean(k * k)
    assert abs(lag1 - 0.9) < 0.02
    assert abs(k.var() - 1 / 64) < 2e-3
    q = x.q.astype(np.float64)[0]
    assert abs(np.mean(q[:, 1:] * q[:, :-1]) / np.mean(q * q)) < 0.02


def test_unit_subset_carries_its_own_state():
    wl = inputs.workload(4, B=2, H=3, T=32)
    x = inputs.make_inputs(wl)
    s = x.units([4, 0])
    assert s.q.shape == (1, 2, 32, 64)
    assert np.array_equal(s.q[0, 0], x.q[1, 1]) and np.array_equal(s.w1[0, 0], x.w1[1])
    assert np.array_equal(s.w2[0, 1], x.w2[0])
