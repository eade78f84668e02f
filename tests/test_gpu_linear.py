"""TTT-Linear: HIP path (through the C ABI) against the fp64 primal oracle.

Sizes: small cases span several 16-token tiles and a ragged tail for every
supported mini-batch shape; the full workloads run on the GPU at their real
size and launch shape and are compared with the oracle element by element
over every (batch, head) unit (the worst unit is printed as a diagnostic).
Edge cases of the method: Theorem 1 ("论文速览 | TTT" §4.1: W0 = 0, eta = 1/2,
b = T is causal linear attention) and eta = 0 (Z = W0 Q, W_T = W0).
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from test_rnn_layers_head_amd import TTTError, inputs, ttt_linear_fwd

pytestmark = pytest.mark.gpu


def small(B, H, T, dtype, seed, eta_dist="sigmoid"):
    wl = inputs.Workload("small", "linear", B=B, H=H, T=T, qkv_dtype=dtype, eta_dist=eta_dist,
                         seed=seed)
    return inputs.make_inputs(wl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 37, 130])
def test_small_parity(dtype, b, T):
    x = small(2, 3, T, dtype, seed=100 + T + b)
    z, w = gu.run_linear(x, b)
    zr, wr = gu.oracle_linear(x, b)
    gu.assert_close(z, zr, dtype, "z")
    gu.assert_close(w, wr, dtype, "w_T")


def test_fp32_workload_full():
    x = inputs.make_inputs(1)
    z, w = gu.run_linear(x, 16)
    zr, wr = gu.oracle_linear(x, 16)
    m = gu.assert_close(z, zr, "f32", "z")
    gu.assert_close(w, wr, "f32", "w_T")
    print("fp32 T=256 z:", m)


def test_125m_workload_full():
    x = inputs.make_inputs(2)
    z, w = gu.run_linear(x, 16)
    zr, wr = gu.oracle_linear(x, 16)
    print("125M z:", gu.assert_close(z, zr, "bf16", "z"), "w:", gu.assert_close(w, wr, "bf16", "w"))


@pytest.fixture(scope="module")
def big():
    return inputs.make_inputs(3)


@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_1p3b_workload_all_units(big, b):
    x = big
    z, w = gu.run_linear(x, b)
    assert np.isfinite(z).all()
    zr, wr = gu.oracle_linear(x, b)
    print(f"1.3B b={b} z:", gu.assert_close_all_units(z, zr, "bf16", "z"),
          "w:", gu.assert_close_all_units(w, wr, "bf16", "w"))


def test_longctx_workload_all_units():
    """The long-context workload in one pass (seq_chunks = 1; the automatic
    choice, chunked, is tested in test_gpu_chunked.py)."""
    x = inputs.make_inputs(5)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    z, w = ttt_linear_fwd(q, k, v, gu.f32(x.eta), gu.f32(x.w0), 16, seq_chunks=1)
    torch.cuda.synchronize()
    z, w = z.cpu().numpy(), w.cpu().numpy()
    zr, wr = gu.oracle_linear(x, 16)
    print("long-ctx z:", gu.assert_close_all_units(z, zr, "bf16", "z"),
          "w:", gu.assert_close_all_units(w, wr, "bf16", "w"))
    # error must not grow along the sequence: compare the last 2k tokens alone
    gu.assert_close(z[:, :, -2048:], zr[:, :, -2048:], "bf16", "z tail")


@pytest.mark.parametrize("b", [16, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_theorem1_causal_linear_attention(dtype, b):
    """W0 = 0, eta = 1/2, one mini-batch of T = b tokens: z_t = sum_{s<=t}
    v_s k_s^T q_t and W_T = sum_s v_s k_s^T, evaluated directly in fp64 from
    the same (rounded) inputs."""
    x = small(2, 3, b, dtype, seed=60 + b)
    x.eta[:] = 0.5
    x.w0[:] = 0.0
    z, w = gu.run_linear(x, b)
    S = np.einsum("bhti,bhtj->bhtij", x.v.astype(np.float64), x.k.astype(np.float64)).cumsum(axis=2)
    zt = np.einsum("bhtij,bhtj->bhti", S, x.q.astype(np.float64))
    gu.assert_close(z, zt, dtype, "z")
    gu.assert_close(w, S[:, :, -1], dtype, "w_T")


@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_eta_zero_leaves_state(b):
    """eta = 0: every update vanishes, so W_T = W0 exactly and Z = W0 Q."""
    x = small(2, 3, 77, "bf16", seed=70 + b)
    x.eta[:] = 0.0
    z, w = gu.run_linear(x, b)
    assert np.array_equal(w, np.broadcast_to(x.w0, w.shape))
    zr = np.einsum("hij,bhtj->bhti", x.w0.astype(np.float64), x.q.astype(np.float64))
    gu.assert_close(z, zr, "bf16", "z")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("b", [4, 16, 32])
def test_row_split_is_bit_identical(dtype, b):
    x = small(3, 5, 77, dtype, seed=7)
    ref = gu.run_linear(x, b, rows=64)
    for rows in (16, 32):
        got = gu.run_linear(x, b, rows=rows)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), rows


@pytest.mark.parametrize("rows", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 16, 37, 300, 2048])
def test_ring_depth_one_is_bit_identical(rows, T):
    """The bf16 scan's LDS prefetch ring only decides when tiles land: one
    tile in flight must give the same bits as the default depth (a missing
    wait would show here as a difference)."""
    x = small(3, 5, T, "bf16", seed=70 + T)
    ref = gu.run_linear(x, 16, rows=rows)
    got = gu.run_linear(x, 16, rows=rows, ring_depth=1)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (rows, T)
    assert np.array_equal(gu.run_linear(x, 16, rows=rows, ring_depth=0)[0], ref[0])


@pytest.mark.parametrize("b, dtype, depth", [(16, "bf16", 2), (8, "bf16", 1), (16, "f32", 1)])
def test_ring_depth_rejections(b, dtype, depth):
    with pytest.raises(TTTError, match="TTT_ERR_UNSUPPORTED"):
        gu.run_linear(small(1, 2, 32, dtype, seed=71), b, ring_depth=depth)


def test_deterministic_reruns():
    x = small(4, 8, 300, "bf16", seed=8)
    a = gu.run_linear(x, 16)
    b = gu.run_linear(x, 16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("b", [4, 16, 64])
def test_state_passing_in_place(b):
    """Two calls, the second resuming in place from the first's final state,
    give the same result as one call (within rounding: the resumed call forms
    its first tile's products directly instead of through the one-tile
    lookahead), and both match the oracle."""
    x = small(2, 4, 320, "bf16", seed=9)
    z, w = gu.run_linear(x, b)
    T1 = 192
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta = gu.f32(x.eta)
    state = gu.f32(np.broadcast_to(x.w0, (2, 4, 64, 64)))
    z1, _ = ttt_linear_fwd(q[:, :, :T1].contiguous(), k[:, :, :T1].contiguous(),
                           v[:, :, :T1].contiguous(), eta[:, :, :T1].contiguous(), state, b,
                           w_out=state)
    z2, _ = ttt_linear_fwd(q[:, :, T1:].contiguous(), k[:, :, T1:].contiguous(),
                           v[:, :, T1:].contiguous(), eta[:, :, T1:].contiguous(), state, b,
                           w_out=state)
    torch.cuda.synchronize()
    z12 = torch.cat([z1, z2], dim=2).cpu().numpy()
    w12 = state.cpu().numpy()
    assert gu.metrics(z12, z)["rel_l2"] < 1e-4 and gu.metrics(w12, w)["rel_l2"] < 1e-4
    zr, wr = gu.oracle_linear(x, b)
    gu.assert_close(z12, zr, "bf16", "z (two calls)")
    gu.assert_close(w12, wr, "bf16", "w (two calls)")
    # the first call alone is bit-identical to the first T1 tokens of one call
    assert np.array_equal(z1.cpu().numpy(), z[:, :, :T1])


def test_side_stream_ordering():
    x = small(2, 2, 64, "bf16", seed=10)
    ref = gu.run_linear(x, 16)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    z = torch.empty((2, 2, 64, 64), device="cuda")
    w = torch.empty((2, 2, 64, 64), device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        z.fill_(float("nan"))
        w.fill_(float("nan"))
        ttt_linear_fwd(q, k, v, eta, w0, 16, z=z, w_out=w, stream=s)
    s.synchronize()
    assert np.array_equal(z.cpu().numpy(), ref[0]) and np.array_equal(w.cpu().numpy(), ref[1])


def test_empty_sequence_copies_state():
    x = small(2, 3, 0, "bf16", seed=11)
    z, w = gu.run_linear(x, 16)
    assert z.shape == (2, 3, 0, 64)
    assert np.array_equal(w, np.broadcast_to(x.w0, w.shape))


def test_empty_batch_is_noop():
    q = torch.empty((0, 3, 16, 64), dtype=torch.bfloat16, device="cuda")
    z, w = ttt_linear_fwd(q, q, q, torch.empty((0, 3, 16), device="cuda"),
                          torch.zeros((3, 64, 64), device="cuda"), 16)
    assert z.numel() == 0 and w.numel() == 0


def test_abi_errors_on_device_tensors():
    x = small(1, 2, 32, "bf16", seed=12)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    with pytest.raises(TTTError) as e:
        ttt_linear_fwd(q, k, v, eta, w0, 3)
    assert e.value.status == 4
    buf = torch.zeros(1 * 2 * 32 * 64, device="cuda")  # z whose storage also holds q
    qa = buf.view(torch.bfloat16)[: 2 * 32 * 64].view(1, 2, 32, 64)
    with pytest.raises(TTTError) as e:
        ttt_linear_fwd(qa, k, v, eta, w0, 16, z=buf.view(1, 2, 32, 64))
    assert e.value.status == 5
    with pytest.raises(TTTError) as e:  # in-place state with a shared initial state
        ttt_linear_fwd(q, k, v, eta, w0, 16, w_out=w0.view(1, 2, 64, 64))
    assert e.value.status == 5
    wmis = torch.zeros(2 * 4096 + 1, device="cuda")[1:].view(2, 64, 64)
    with pytest.raises(TTTError) as e:
        ttt_linear_fwd(q, k, v, eta, wmis, 16)
    assert e.value.status == 7
