"""Helpers for GPU parity tests (not collected): device copies of the seeded
inputs and the error metrics the tolerances are stated in."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle

# Tolerances: rel-L2 <= 1e-5 for fp32 inputs; for bf16 inputs rel-L2 <= 2e-3
# and max|diff| / RMS(reference) <= 1e-2, applied to Z and the final state.
TOL_F32_REL = 1e-5
TOL_BF16_REL = 2e-3
TOL_BF16_MAX = 1e-2


def dev(x, name):
    """Device tensor of an input array in its storage format."""
    a = getattr(x, name + "_raw")
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    rms = np.sqrt(np.mean(ref * ref))
    return {
        "rel_l2": float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)),
        "max_over_rms": float(np.abs(diff).max() / max(rms, 1e-300)) if diff.size else 0.0,
    }


def assert_close(got, ref, qkv_dtype, what=""):
    m = metrics(got, ref)
    if qkv_dtype == "f32":
        assert m["rel_l2"] <= TOL_F32_REL, (what, m)
    else:
        assert m["rel_l2"] <= TOL_BF16_REL and m["max_over_rms"] <= TOL_BF16_MAX, (what, m)
    return m


def worst_unit(got, ref):
    """Diagnostic: the (batch, head) unit with the largest relative L2 error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(got.shape[0] * got.shape[1], -1)
    r = ref.reshape(g.shape)
    e = np.linalg.norm(g - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    u = int(np.argmax(e)) if e.size else -1
    return {"unit": u, "rel_l2": float(e[u]) if e.size else 0.0}


def assert_close_all_units(got, ref, qkv_dtype, what=""):
    """Whole-tensor tolerance check plus the worst unit's error (printed)."""
    m = assert_close(got, ref, qkv_dtype, what)
    m["worst_unit"] = worst_unit(got, ref)
    return m


def oracle_units_parallel(fn, n_units, threads=None):
    """Runs fn(unit_index) for every unit on a thread pool (the oracle's C
    calls release the GIL) and returns the results in unit order."""
    from concurrent.futures import ThreadPoolExecutor
    threads = threads or oracle.default_threads()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, range(n_units)))


def run_linear(x, b, rows=0, ring_depth=None):
    from test_rnn_layers_head_amd import ttt_linear_fwd
    z, w = ttt_linear_fwd(dev(x, "q"), dev(x, "k"), dev(x, "v"), f32(x.eta), f32(x.w0), b,
                          rows_per_workgroup=rows, ring_depth=ring_depth)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w.cpu().numpy()


def oracle_linear(x, b):
    return oracle.linear(x.q, x.k, x.v, x.eta, x.w0, b)


def run_mlp(x, b):
    from test_rnn_layers_head_amd import ttt_mlp_fwd
    z, w1, w2 = ttt_mlp_fwd(dev(x, "q"), dev(x, "k"), dev(x, "v"), f32(x.eta), f32(x.w1),
                            f32(x.w2), b)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w1.cpu().numpy(), w2.cpu().numpy()


def oracle_mlp(x, b):
    return oracle.mlp(x.q, x.k, x.v, x.eta, x.w1, x.w2, b)


def run_linear_ln(x, b, gamma=None, beta=None, eps=None, w0=None):
    from test_rnn_layers_head_amd import ttt_linear_ln_fwd
    gamma = x.ln_gamma if gamma is None else gamma
    beta = x.ln_beta if beta is None else beta
    eps = x.wl.ln_eps if eps is None else eps
    w0 = x.w0 if w0 is None else w0
    z, w = ttt_linear_ln_fwd(dev(x, "q"), dev(x, "k"), dev(x, "v"), f32(x.eta), f32(w0),
                             f32(gamma), f32(beta), eps, b)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w.cpu().numpy()


def oracle_linear_ln(x, b, gamma=None, beta=None, eps=None, w0=None):
    gamma = x.ln_gamma if gamma is None else gamma
    beta = x.ln_beta if beta is None else beta
    eps = x.wl.ln_eps if eps is None else eps
    w0 = x.w0 if w0 is None else w0
    return oracle.linear_ln(x.q, x.k, x.v, x.eta, w0, gamma, beta, eps, b)
