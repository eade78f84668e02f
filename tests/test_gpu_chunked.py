"""The chunked (sequence-parallel) TTT-Linear scan against the fp64 oracle.

Each mini-batch maps the state affinely (W -> W (I - 2 K D K^T) + 2 V D K^T),
so the scan can run every sequence chunk's map at once, chain the maps and
rerun the chunks from their start states.  These cases force the chunk
count through ttt_linear_fwd_chunked, check the automatic choice of
ttt_linear_fwd, and check that z's prior contents (the passes keep their
intermediate states there) never reach the results.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from test_rnn_layers_head_amd import TTTError, inputs, ttt_linear_fwd, ttt_linear_fwd_plan

pytestmark = pytest.mark.gpu


def case(B, H, T, seed, eta_dist="sigmoid"):
    wl = inputs.Workload("chunked", "linear", B=B, H=H, T=T, eta_dist=eta_dist, seed=seed)
    return inputs.make_inputs(wl)


def run(x, P, rows=0, w0=None, poison=True):
    q, k, v = (gu.dev(x, n) for n in "qkv")
    B, H, T = x.wl.B, x.wl.H, x.wl.T
    z = torch.full((B, H, T, 64), float("nan") if poison else 0.0, device="cuda")
    w0 = gu.f32(x.w0) if w0 is None else w0
    zz, w = ttt_linear_fwd(q, k, v, gu.f32(x.eta), w0, 16, z=z, rows_per_workgroup=rows,
                           seq_chunks=P)
    torch.cuda.synchronize()
    return zz.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("B,H,T,P,rows", [
    (1, 2, 1024, 4, 0),     # 256-token chunks, the shortest allowed is 192
    (2, 2, 768, 2, 16),
    (1, 3, 2048, 8, 32),
    (1, 1, 4096, 16, 64),
    (2, 1, 960, 5, 0),      # an odd chunk count: 192-token chunks
])
def test_chunked_matches_oracle(B, H, T, P, rows):
    x = case(B, H, T, seed=400 + P + rows)
    z, w = run(x, P, rows)
    zr, wr = gu.oracle_linear(x, 16)
    mz = gu.assert_close(z, zr, "bf16", "z")
    mw = gu.assert_close(w, wr, "bf16", "w_T")
    # the single pass over the same inputs: equal up to rounding order
    z1, w1 = run(x, 1, rows)
    assert gu.metrics(z, z1)["rel_l2"] < 1e-5 and gu.metrics(w, w1)["rel_l2"] < 1e-5
    print(f"P={P} rows={rows} z:", mz, "w:", mw)


def test_chunked_is_deterministic_and_ignores_prior_z():
    x = case(1, 2, 1024, seed=411)
    a = run(x, 4, poison=True)
    b = run(x, 4, poison=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_chunked_in_place_resume():
    """w0_per_batch = 1 with w_out the same tensor as w0: the start state is
    read before the final state is written."""
    x = case(2, 2, 1024, seed=412)
    state = gu.f32(np.broadcast_to(x.w0, (2, 2, 64, 64)))
    z, w = run(x, 4, w0=state)
    zr, wr = gu.oracle_linear(x, 16)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    z2, _ = ttt_linear_fwd(q, k, v, gu.f32(x.eta), state, 16, w_out=state, seq_chunks=4)
    torch.cuda.synchronize()
    gu.assert_close(z2.cpu().numpy(), zr, "bf16", "z (in place)")
    gu.assert_close(state.cpu().numpy(), wr, "bf16", "w (in place)")
    assert np.array_equal(z2.cpu().numpy(), z) and np.array_equal(state.cpu().numpy(), w)


def test_automatic_choice_chunks_few_long_sequences():
    """ttt_linear_fwd cuts 2 units of 8192 tokens into 8 chunks, and runs one
    pass for 128 units of 2048 tokens and for 32 units of 4096."""
    assert ttt_linear_fwd_plan(1, 2, 8192, 16) == (16, 8)
    assert ttt_linear_fwd_plan(8, 16, 2048, 16)[1] == 1 and ttt_linear_fwd_plan(2, 16, 4096, 16)[1] == 1
    x = case(1, 2, 8192, seed=413)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    z, w = ttt_linear_fwd(q, k, v, gu.f32(x.eta), gu.f32(x.w0), 16)
    torch.cuda.synchronize()
    z8, w8 = run(x, 8, poison=False)
    assert np.array_equal(z.cpu().numpy(), z8) and np.array_equal(w.cpu().numpy(), w8)
    z1, _ = run(x, 1, poison=False)
    assert not np.array_equal(z8, z1)  # the chunked passes ran
    zr, wr = gu.oracle_linear(x, 16)
    gu.assert_close(z8, zr, "bf16", "z")
    gu.assert_close(w8, wr, "bf16", "w")
    for (B, H, T) in [(8, 16, 2048), (2, 16, 4096)]:
        y = case(B, H, T, seed=414 + T)
        qy, ky, vy = (gu.dev(y, n) for n in "qkv")
        za, _ = ttt_linear_fwd(qy, ky, vy, gu.f32(y.eta), gu.f32(y.w0), 16)
        torch.cuda.synchronize()
        zb, _ = run(y, 1, poison=False)
        assert np.array_equal(za.cpu().numpy(), zb), (B, H, T)


def test_long_context_workload_chunked_all_units():
    """The long-context workload (1 x 32 x 32768) takes the chunked path:
    every unit against the oracle, over the whole sequence and its end."""
    x = inputs.make_inputs(5)
    z, w = run(x, 8, poison=False)
    zr, wr = gu.oracle_linear(x, 16)
    print("long-ctx chunked z:", gu.assert_close_all_units(z, zr, "bf16", "z"),
          "w:", gu.assert_close_all_units(w, wr, "bf16", "w"))
    gu.assert_close(z[:, :, -2048:], zr[:, :, -2048:], "bf16", "z tail")


@pytest.mark.parametrize("kw", [
    dict(T=1024, P=3),        # T not a multiple of P
    dict(T=512, P=4),         # 128-token chunks
    dict(T=1000, P=2),        # 500-token chunks, not a multiple of 16
])
def test_chunked_rejects_unsupported_splits(kw):
    x = case(1, 1, kw["T"], seed=415)
    with pytest.raises(TTTError) as e:
        run(x, kw["P"])
    assert e.value.status == 4


def test_chunked_graph_replays_match_eager():
    """The chunked scan's four launches captured in one HIP graph: every
    replay gives exactly the eager result (z starts NaN-filled each time)."""
    x = case(1, 2, 2048, seed=416)
    q, k, v = (gu.dev(x, n) for n in "qkv")
    eta, w0 = gu.f32(x.eta), gu.f32(x.w0)
    ze, we = ttt_linear_fwd(q, k, v, eta, w0, 16, seq_chunks=8)
    torch.cuda.synchronize()
    z, w = torch.empty_like(ze), torch.empty_like(we)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ttt_linear_fwd(q, k, v, eta, w0, 16, z=z, w_out=w, seq_chunks=8)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        z.fill_(float("nan"))
        w.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 16, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        assert torch.equal(z, ze) and torch.equal(w, we), rep
        assert torch.isfinite(scratch)
