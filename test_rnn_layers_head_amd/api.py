"""Python binding of the TTT scan C ABI over torch tensors.

Argument marshalling only: shapes, dtypes and the current HIP stream are read
from the tensors and passed to libttt.so; every step of the scan runs in the
HIP kernels.  Tensors must live on a GPU; there is no CPU path.
"""
from __future__ import annotations

import torch

from . import _lib


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.TTT_BF16
    if t.dtype == torch.float32:
        return _lib.TTT_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check_tensors(named: dict) -> torch.device:
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got {t.device}); the scan runs only "
                             "in the HIP kernels")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def _stream(dev, stream):
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def ttt_linear_fwd_plan(B: int, H: int, T: int, b: int, dtype=torch.bfloat16):
    """(rows_per_workgroup, seq_chunks) that ttt_linear_fwd picks for these
    sizes (ttt_tuning.h); host-only."""
    import ctypes
    rows, chunks = ctypes.c_int32(0), ctypes.c_int32(0)
    code = _lib.TTT_BF16 if dtype == torch.bfloat16 else _lib.TTT_F32
    _lib.check(_lib.lib().ttt_linear_fwd_plan(int(B), int(H), int(T), int(b), code,
                                               ctypes.addressof(rows), ctypes.addressof(chunks)))
    return rows.value, chunks.value


def ttt_linear_fwd(q, k, v, eta, w0, b: int, z=None, w_out=None, stream=None,
                   rows_per_workgroup: int = 0, seq_chunks=None, ring_depth=None):
    """TTT-Linear forward scan (see include/ttt.h).

    q, k, v: [B, H, T, d] bf16 or fp32; eta: [B, H, T] fp32; w0: [H, d, d] or
    [B, H, d, d] fp32.  Outputs z [B, H, T, d] fp32 and w_out [B, H, d, d]
    fp32 are allocated when not given.  Returns (z, w_out).
    rows_per_workgroup (ttt_linear_fwd_tuned) and seq_chunks
    (ttt_linear_fwd_chunked) select the launch shape; by default the library
    picks both.  ring_depth (ttt_linear_fwd_ring_depth: 0 default, 1 one tile
    in flight) sets the bf16 scan's LDS prefetch depth.
    """
    B, H, T, d = q.shape
    if z is None:
        z = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if w_out is None:
        w_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w0=w0, z=z, w_out=w_out))
    for name, t in (("eta", eta), ("w0", w0), ("z", z), ("w_out", w_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if k.shape != q.shape or v.shape != q.shape or tuple(eta.shape) != (B, H, T):
        raise ValueError("shape mismatch among q, k, v, eta")
    per_batch = 1 if w0.dim() == 4 else 0
    if tuple(w0.shape) != ((B, H, d, d) if per_batch else (H, d, d)):
        raise ValueError(f"w0 has shape {tuple(w0.shape)}")
    if tuple(z.shape) != (B, H, T, d) or tuple(w_out.shape) != (B, H, d, d):
        raise ValueError("output shape mismatch")
    L = _lib.lib()
    with torch.cuda.device(dev):
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch, B, H, T, d, int(b),
                _dtype_code(q), _ptr(z), _ptr(w_out), _stream(dev, stream))
        if ring_depth is not None:
            _lib.check(L.ttt_linear_fwd_ring_depth(*args, int(rows_per_workgroup),
                                                   int(ring_depth)))
        elif seq_chunks is not None:
            _lib.check(L.ttt_linear_fwd_chunked(*args, int(rows_per_workgroup), int(seq_chunks)))
        elif rows_per_workgroup:
            _lib.check(L.ttt_linear_fwd_tuned(*args, int(rows_per_workgroup)))
        else:
            _lib.check(L.ttt_linear_fwd(*args))
    return z, w_out


def ttt_linear_ln_fwd(q, k, v, eta, w0, ln_gamma, ln_beta, eps: float, b: int, z=None,
                      w_out=None, stream=None):
    """TTT-Linear with the LayerNorm + residual inner model, f(x) = x + LN(W x)
    (see include/ttt.h).

    q, k, v: [B, H, T, d] bf16 or fp32; eta: [B, H, T] fp32; w0: [H, d, d] or
    [B, H, d, d] fp32; ln_gamma, ln_beta: [H, d] fp32; eps > 0.  Returns
    (z, w_out), allocated when not given.
    """
    B, H, T, d = q.shape
    if z is None:
        z = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if w_out is None:
        w_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w0=w0, ln_gamma=ln_gamma, ln_beta=ln_beta,
                              z=z, w_out=w_out))
    for name, t in (("eta", eta), ("w0", w0), ("ln_gamma", ln_gamma), ("ln_beta", ln_beta),
                    ("z", z), ("w_out", w_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if k.shape != q.shape or v.shape != q.shape or tuple(eta.shape) != (B, H, T):
        raise ValueError("shape mismatch among q, k, v, eta")
    per_batch = 1 if w0.dim() == 4 else 0
    if tuple(w0.shape) != ((B, H, d, d) if per_batch else (H, d, d)):
        raise ValueError(f"w0 has shape {tuple(w0.shape)}")
    if tuple(ln_gamma.shape) != (H, d) or tuple(ln_beta.shape) != (H, d):
        raise ValueError("ln_gamma / ln_beta must be [H, d]")
    if tuple(z.shape) != (B, H, T, d) or tuple(w_out.shape) != (B, H, d, d):
        raise ValueError("output shape mismatch")
    L = _lib.lib()
    with torch.cuda.device(dev):
        _lib.check(L.ttt_linear_ln_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch,
                                       _ptr(ln_gamma), _ptr(ln_beta), float(eps), B, H, T, d,
                                       int(b), _dtype_code(q), _ptr(z), _ptr(w_out),
                                       _stream(dev, stream)))
    return z, w_out


def ttt_linear_ln_fwd_ckpt(q, k, v, eta, w0, ln_gamma, ln_beta, eps: float, b: int, stream=None):
    """ttt_linear_ln_fwd that also keeps the state before every mini-batch
    (include/ttt.h).  Returns (z, w_out, w_ckpt), w_ckpt [B, H, ceil(T/b), d, d]."""
    B, H, T, d = q.shape
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    z, w_out = f32(B, H, T, d), f32(B, H, d, d)
    w_ckpt = f32(B, H, (T + b - 1) // b if b > 0 else 0, d, d)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w0=w0, ln_gamma=ln_gamma, ln_beta=ln_beta))
    for name, t in (("eta", eta), ("w0", w0), ("ln_gamma", ln_gamma), ("ln_beta", ln_beta)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    per_batch = 1 if w0.dim() == 4 else 0
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_linear_ln_fwd_ckpt(
            _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0), per_batch, _ptr(ln_gamma),
            _ptr(ln_beta), float(eps), B, H, T, d, int(b), _dtype_code(q), _ptr(z), _ptr(w_out),
            _ptr(w_ckpt), _stream(dev, stream)))
    return z, w_out, w_ckpt


def ttt_linear_ln_bwd(q, k, v, eta, w_ckpt, ln_gamma, ln_beta, eps: float, b: int, dz, dw_T=None,
                      stream=None):
    """Backward of TTT-Linear with the LayerNorm + residual inner model
    (include/ttt.h): returns (dq, dk, dv, deta, dw0, dgamma, dbeta), fp32,
    with dw0 [B, H, d, d] and dgamma, dbeta [B, H, d] per unit."""
    B, H, T, d = q.shape
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    dq, dk, dv, deta = f32(B, H, T, d), f32(B, H, T, d), f32(B, H, T, d), f32(B, H, T)
    dw0, dg, db = f32(B, H, d, d), f32(B, H, d), f32(B, H, d)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w_ckpt=w_ckpt, ln_gamma=ln_gamma,
                              ln_beta=ln_beta, dz=dz, dw_T=dw_T))
    for name, t in (("dz", dz), ("dw_T", dw_T), ("w_ckpt", w_ckpt), ("eta", eta)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if tuple(dz.shape) != (B, H, T, d):
        raise ValueError("dz must be [B, H, T, d]")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_linear_ln_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w_ckpt), _ptr(ln_gamma), _ptr(ln_beta),
            float(eps), B, H, T, d, int(b), _dtype_code(q), _ptr(dz), _ptr(dw_T), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0), _ptr(dg), _ptr(db), _stream(dev, stream)))
    return dq, dk, dv, deta, dw0, dg, db


def ttt_linear_fwd_ckpt(q, k, v, eta, w0, b: int, z=None, w_out=None, w_ckpt=None, stream=None):
    """ttt_linear_fwd that also keeps the state before every mini-batch
    (include/ttt.h).  Returns (z, w_out, w_ckpt) with w_ckpt
    [B, H, ceil(T/b), d, d] fp32."""
    B, H, T, d = q.shape
    nmb = (T + b - 1) // b if b > 0 else 0
    if w_ckpt is None:
        w_ckpt = torch.empty((B, H, nmb, d, d), dtype=torch.float32, device=q.device)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if w_out is None:
        w_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w0=w0, z=z, w_out=w_out, w_ckpt=w_ckpt))
    if tuple(w_ckpt.shape) != (B, H, nmb, d, d) or w_ckpt.dtype != torch.float32:
        raise ValueError("w_ckpt must be float32 [B, H, ceil(T/b), d, d]")
    per_batch = 1 if w0.dim() == 4 else 0
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_linear_fwd_ckpt(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w0),
                                                  per_batch, B, H, T, d, int(b), _dtype_code(q),
                                                  _ptr(z), _ptr(w_out), _ptr(w_ckpt),
                                                  _stream(dev, stream)))
    return z, w_out, w_ckpt


def ttt_linear_bwd(q, k, v, eta, w_ckpt, b: int, dz, dw_T=None, stream=None, seq_chunks=None):
    """Backward of the TTT-Linear scan (include/ttt.h): given dz = dL/dZ and
    optionally dw_T = dL/dW_T, returns (dq, dk, dv, deta, dw0), fp32, with
    dw0 per unit [B, H, d, d].  w_ckpt comes from ttt_linear_fwd_ckpt.
    seq_chunks: None or 0 = automatic, 1 = one pass, P >= 2 = P sequence
    chunks (ttt_linear_bwd_chunked, ttt_tuning.h)."""
    B, H, T, d = q.shape
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    dq, dk, dv, deta, dw0 = f32(B, H, T, d), f32(B, H, T, d), f32(B, H, T, d), f32(B, H, T), \
        f32(B, H, d, d)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w_ckpt=w_ckpt, dz=dz, dw_T=dw_T))
    for name, t in (("dz", dz), ("dw_T", dw_T), ("w_ckpt", w_ckpt)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if tuple(dz.shape) != (B, H, T, d):
        raise ValueError("dz must be [B, H, T, d]")
    if b > 0 and tuple(w_ckpt.shape) != (B, H, (T + b - 1) // b, d, d):
        raise ValueError("w_ckpt must be [B, H, ceil(T/b), d, d]")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w_ckpt), B, H, T, d, int(b), _dtype_code(q),
            _ptr(dz), _ptr(dw_T), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dw0))
    with torch.cuda.device(dev):
        if seq_chunks is None:
            _lib.check(_lib.lib().ttt_linear_bwd(*args, _stream(dev, stream)))
        else:
            _lib.check(_lib.lib().ttt_linear_bwd_chunked(*args, _stream(dev, stream), int(seq_chunks)))
    return dq, dk, dv, deta, dw0


def _step_common(name, q, k, v, eta, pos, states: dict, z):
    if q.dim() != 3:
        raise ValueError(f"{name}: q must be [B, H, d] (one token per unit)")
    B, H, d = q.shape
    if z is None:
        z = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, pos=pos, z=z, **states))
    for nm, t in (("eta", eta), ("z", z), *states.items()):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32, got {t.dtype}")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,):
        raise TypeError("pos must be an int32 tensor of shape [B]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if k.shape != q.shape or v.shape != q.shape or tuple(eta.shape) != (B, H):
        raise ValueError("shape mismatch among q, k, v, eta")
    if tuple(z.shape) != (B, H, d):
        raise ValueError("z must be [B, H, d]")
    return B, H, d, z, dev


def ttt_linear_step(q, k, v, eta, w, w_gp, pos, b: int, z=None, stream=None):
    """One TTT-Linear decode step for every (batch, head) unit (include/ttt.h).

    q, k, v: [B, H, d] (this token); eta: [B, H] fp32; w, w_gp: [B, H, d, d]
    fp32, the state and the gradient point, updated in place (w_gp may be
    None when b == 1); pos: [B] int32, the token's index in its sequence.
    Returns z [B, H, d] fp32.
    """
    B, H, d, z, dev = _step_common("ttt_linear_step", q, k, v, eta, pos, dict(w=w, w_gp=w_gp), z)
    for nm, t in (("w", w), ("w_gp", w_gp)):
        if t is not None and tuple(t.shape) != (B, H, d, d):
            raise ValueError(f"{nm} must be [B, H, d, d]")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_linear_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w),
                                              _ptr(w_gp), _ptr(pos), B, H, d, int(b),
                                              _dtype_code(q), _ptr(z), _stream(dev, stream)))
    return z


def ttt_linear_ln_step(q, k, v, eta, w, w_gp, pos, ln_gamma, ln_beta, eps: float, b: int, z=None,
                       stream=None):
    """One decode step of TTT-Linear with the LayerNorm + residual inner
    model; as ttt_linear_step plus ln_gamma, ln_beta [H, d] fp32 and eps."""
    B, H, d, z, dev = _step_common("ttt_linear_ln_step", q, k, v, eta, pos,
                                   dict(w=w, w_gp=w_gp, ln_gamma=ln_gamma, ln_beta=ln_beta), z)
    for nm, t in (("w", w), ("w_gp", w_gp)):
        if t is not None and tuple(t.shape) != (B, H, d, d):
            raise ValueError(f"{nm} must be [B, H, d, d]")
    if tuple(ln_gamma.shape) != (H, d) or tuple(ln_beta.shape) != (H, d):
        raise ValueError("ln_gamma / ln_beta must be [H, d]")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_linear_ln_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w),
                                                 _ptr(w_gp), _ptr(pos), _ptr(ln_gamma),
                                                 _ptr(ln_beta), float(eps), B, H, d, int(b),
                                                 _dtype_code(q), _ptr(z), _stream(dev, stream)))
    return z


def ttt_mlp_step(q, k, v, eta, w1, w2, w1_gp, w2_gp, pos, b: int, z=None, stream=None):
    """One TTT-MLP decode step (include/ttt.h): w1, w1_gp [B, H, hidden, d],
    w2, w2_gp [B, H, d, hidden] fp32, updated in place (the gradient points
    may be None when b == 1).  Returns z [B, H, d] fp32."""
    B, H, d, z, dev = _step_common("ttt_mlp_step", q, k, v, eta, pos,
                                   dict(w1=w1, w2=w2, w1_gp=w1_gp, w2_gp=w2_gp), z)
    hidden = w1.shape[-2]
    for nm, t, shp in (("w1", w1, (B, H, hidden, d)), ("w2", w2, (B, H, d, hidden)),
                       ("w1_gp", w1_gp, (B, H, hidden, d)), ("w2_gp", w2_gp, (B, H, d, hidden))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{nm} must be {list(shp)}")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_mlp_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1), _ptr(w2),
                                           _ptr(w1_gp), _ptr(w2_gp), _ptr(pos), B, H, d, hidden,
                                           int(b), _dtype_code(q), _ptr(z), _stream(dev, stream)))
    return z


def ttt_mlp_fwd(q, k, v, eta, w1_0, w2_0, b: int, z=None, w1_out=None, w2_out=None, stream=None):
    """TTT-MLP forward scan, f(x) = W2 GELU(W1 x) (see include/ttt.h).

    w1_0: [H, hidden, d] or [B, H, hidden, d]; w2_0: [H, d, hidden] or
    [B, H, d, hidden] (fp32).  Returns (z, w1_out, w2_out).
    """
    B, H, T, d = q.shape
    hidden = w1_0.shape[-2]
    if z is None:
        z = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if w1_out is None:
        w1_out = torch.empty((B, H, hidden, d), dtype=torch.float32, device=q.device)
    if w2_out is None:
        w2_out = torch.empty((B, H, d, hidden), dtype=torch.float32, device=q.device)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w1_0=w1_0, w2_0=w2_0, z=z, w1_out=w1_out,
                              w2_out=w2_out))
    for name, t in (("eta", eta), ("w1_0", w1_0), ("w2_0", w2_0), ("z", z), ("w1_out", w1_out),
                    ("w2_out", w2_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    per_batch = 1 if w1_0.dim() == 4 else 0
    lead = (B, H) if per_batch else (H,)
    if tuple(w1_0.shape) != (*lead, hidden, d) or tuple(w2_0.shape) != (*lead, d, hidden):
        raise ValueError("w1_0 / w2_0 shape mismatch")
    L = _lib.lib()
    with torch.cuda.device(dev):
        _lib.check(L.ttt_mlp_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_0), _ptr(w2_0),
                                 per_batch, B, H, T, d, hidden, int(b), _dtype_code(q), _ptr(z),
                                 _ptr(w1_out), _ptr(w2_out), _stream(dev, stream)))
    return z, w1_out, w2_out


def ttt_mlp_ln_fwd(q, k, v, eta, w1_0, w2_0, ln_gamma, ln_beta, eps: float, b: int, z=None,
                   w1_out=None, w2_out=None, stream=None):
    """TTT-MLP with the LayerNorm + residual wrapper,
    f(x) = x + LN(W2 GELU(W1 x)) (see include/ttt.h).

    Arguments as for ttt_mlp_fwd, plus ln_gamma, ln_beta: [H, d] fp32 and
    eps > 0.  Returns (z, w1_out, w2_out), allocated when not given.
    """
    B, H, T, d = q.shape
    hidden = w1_0.shape[-2]
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    z = f32(B, H, T, d) if z is None else z
    w1_out = f32(B, H, hidden, d) if w1_out is None else w1_out
    w2_out = f32(B, H, d, hidden) if w2_out is None else w2_out
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w1_0=w1_0, w2_0=w2_0, ln_gamma=ln_gamma,
                              ln_beta=ln_beta, z=z, w1_out=w1_out, w2_out=w2_out))
    for name, t in (("eta", eta), ("w1_0", w1_0), ("w2_0", w2_0), ("ln_gamma", ln_gamma),
                    ("ln_beta", ln_beta), ("z", z), ("w1_out", w1_out), ("w2_out", w2_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if tuple(ln_gamma.shape) != (H, d) or tuple(ln_beta.shape) != (H, d):
        raise ValueError("ln_gamma / ln_beta must be [H, d]")
    per_batch = 1 if w1_0.dim() == 4 else 0
    lead = (B, H) if per_batch else (H,)
    if tuple(w1_0.shape) != (*lead, hidden, d) or tuple(w2_0.shape) != (*lead, d, hidden):
        raise ValueError("w1_0 / w2_0 shape mismatch")
    L = _lib.lib()
    with torch.cuda.device(dev):
        _lib.check(L.ttt_mlp_ln_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_0), _ptr(w2_0),
                                    per_batch, _ptr(ln_gamma), _ptr(ln_beta), float(eps), B, H, T,
                                    d, hidden, int(b), _dtype_code(q), _ptr(z), _ptr(w1_out),
                                    _ptr(w2_out), _stream(dev, stream)))
    return z, w1_out, w2_out


def ttt_mlp_fwd_ckpt(q, k, v, eta, w1_0, w2_0, b: int, z=None, w1_out=None, w2_out=None,
                     w1_ckpt=None, w2_ckpt=None, stream=None):
    """ttt_mlp_fwd that also keeps both layers' state before every mini-batch
    of b tokens (include/ttt.h).  Returns (z, w1_out, w2_out, w1_ckpt,
    w2_ckpt) with w1_ckpt [B, H, ceil(T/b), hidden, d] and w2_ckpt
    [B, H, ceil(T/b), d, hidden], fp32."""
    B, H, T, d = q.shape
    hidden = w1_0.shape[-2]
    nmb = (T + b - 1) // b if b > 0 else 0
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    z = f32(B, H, T, d) if z is None else z
    w1_out = f32(B, H, hidden, d) if w1_out is None else w1_out
    w2_out = f32(B, H, d, hidden) if w2_out is None else w2_out
    w1_ckpt = f32(B, H, nmb, hidden, d) if w1_ckpt is None else w1_ckpt
    w2_ckpt = f32(B, H, nmb, d, hidden) if w2_ckpt is None else w2_ckpt
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w1_0=w1_0, w2_0=w2_0, z=z, w1_out=w1_out,
                              w2_out=w2_out, w1_ckpt=w1_ckpt, w2_ckpt=w2_ckpt))
    for name, t in (("eta", eta), ("w1_0", w1_0), ("w2_0", w2_0), ("z", z), ("w1_out", w1_out),
                    ("w2_out", w2_out), ("w1_ckpt", w1_ckpt), ("w2_ckpt", w2_ckpt)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if tuple(w1_ckpt.shape) != (B, H, nmb, hidden, d) or tuple(w2_ckpt.shape) != (B, H, nmb, d, hidden):
        raise ValueError("w1_ckpt / w2_ckpt must be [B, H, ceil(T/b), hidden, d] / [.., d, hidden]")
    per_batch = 1 if w1_0.dim() == 4 else 0
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_mlp_fwd_ckpt(
            _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_0), _ptr(w2_0), per_batch, B, H, T, d,
            hidden, int(b), _dtype_code(q), _ptr(z), _ptr(w1_out), _ptr(w2_out), _ptr(w1_ckpt),
            _ptr(w2_ckpt), _stream(dev, stream)))
    return z, w1_out, w2_out, w1_ckpt, w2_ckpt


def ttt_mlp_bwd(q, k, v, eta, w1_ckpt, w2_ckpt, b: int, dz, dw1_T=None, dw2_T=None, stream=None):
    """Backward of the TTT-MLP scan (include/ttt.h): given dz = dL/dZ and
    optionally the adjoints of the final states, returns (dq, dk, dv, deta,
    dw1_0, dw2_0), fp32, with the initial-state adjoints per unit.  The
    checkpoints come from ttt_mlp_fwd_ckpt with the same b."""
    B, H, T, d = q.shape
    hidden = w1_ckpt.shape[-2]
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    dq, dk, dv, deta = f32(B, H, T, d), f32(B, H, T, d), f32(B, H, T, d), f32(B, H, T)
    dw1, dw2 = f32(B, H, hidden, d), f32(B, H, d, hidden)
    dev = _check_tensors(dict(q=q, k=k, v=v, eta=eta, w1_ckpt=w1_ckpt, w2_ckpt=w2_ckpt, dz=dz,
                              dw1_T=dw1_T, dw2_T=dw2_T))
    for name, t in (("dz", dz), ("dw1_T", dw1_T), ("dw2_T", dw2_T), ("w1_ckpt", w1_ckpt),
                    ("w2_ckpt", w2_ckpt), ("eta", eta)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if tuple(dz.shape) != (B, H, T, d):
        raise ValueError("dz must be [B, H, T, d]")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_mlp_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(w1_ckpt), _ptr(w2_ckpt), B, H, T, d, hidden,
            int(b), _dtype_code(q), _ptr(dz), _ptr(dw1_T), _ptr(dw2_T), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(deta), _ptr(dw1), _ptr(dw2), _stream(dev, stream)))
    return dq, dk, dv, deta, dw1, dw2


def _gate_common(x, theta_lr, H_expected, eta):
    if x.dim() != 3:
        raise ValueError("x must be [B, T, dx]")
    if x.dtype != torch.bfloat16:
        raise TypeError(f"x must be bfloat16, got {x.dtype}")
    if theta_lr.dtype != torch.float32:
        raise TypeError(f"theta_lr must be float32, got {theta_lr.dtype}")
    B, T, dx = x.shape
    H = theta_lr.shape[0] if H_expected is None else H_expected
    if tuple(theta_lr.shape) != (H, dx):
        raise ValueError(f"theta_lr must be [H, dx] = [{H}, {dx}], got {tuple(theta_lr.shape)}")
    if eta is None:
        eta = torch.empty((B, H, T), dtype=torch.float32, device=x.device)
    if eta.dtype != torch.float32 or tuple(eta.shape) != (B, H, T):
        raise ValueError("eta must be float32 [B, H, T]")
    return B, T, H, dx, eta


def ttt_lr_gate(x, theta_lr, eta_base: float, eta=None, stream=None, tokens_per_workgroup: int = 0):
    """Learning-rate gate (include/ttt.h): x [B, T, dx] bf16, theta_lr
    [H, dx] fp32 -> eta [B, H, T] = eta_base * sigmoid(theta_lr[h] . x[b, t])."""
    B, T, H, dx, eta = _gate_common(x, theta_lr, None, eta)
    dev = _check_tensors(dict(x=x, theta_lr=theta_lr, eta=eta))
    L = _lib.lib()
    with torch.cuda.device(dev):
        args = (_ptr(x), _lib.TTT_BF16, _ptr(theta_lr), float(eta_base), B, T, H, dx, _ptr(eta),
                _stream(dev, stream))
        if tokens_per_workgroup:
            _lib.check(L.ttt_lr_gate_tuned(*args, int(tokens_per_workgroup)))
        else:
            _lib.check(L.ttt_lr_gate(*args))
    return eta


def ttt_lr_gate_bwd(x, theta_lr, eta_base: float, eta, deta, dtheta_lr=None, dx=None, stream=None):
    """Backward of the learning-rate gate (include/ttt.h): deta = dL/deta
    [B, H, T] and the gate's output eta -> (dtheta_lr [H, dx], dx [B, T, dx]),
    fp32."""
    B, T, H, d_x, _ = _gate_common(x, theta_lr, None, eta)
    for name, t in (("deta", deta),):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, T):
            raise ValueError(f"{name} must be float32 [B, H, T]")
    if dtheta_lr is None:
        dtheta_lr = torch.empty((H, d_x), dtype=torch.float32, device=x.device)
    if dx is None:
        dx = torch.empty((B, T, d_x), dtype=torch.float32, device=x.device)
    if dtheta_lr.dtype != torch.float32 or tuple(dtheta_lr.shape) != (H, d_x):
        raise ValueError("dtheta_lr must be float32 [H, dx]")
    if dx.dtype != torch.float32 or tuple(dx.shape) != (B, T, d_x):
        raise ValueError("dx must be float32 [B, T, dx]")
    dev = _check_tensors(dict(x=x, theta_lr=theta_lr, eta=eta, deta=deta, dtheta_lr=dtheta_lr,
                              dx=dx))
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_lr_gate_bwd(_ptr(x), _lib.TTT_BF16, _ptr(theta_lr),
                                              float(eta_base), _ptr(eta), _ptr(deta), B, T, H,
                                              d_x, _ptr(dtheta_lr), _ptr(dx), _stream(dev, stream)))
    return dtheta_lr, dx


def ttt_linear_gated_fwd(q, k, v, x, theta_lr, eta_base: float, w0, b: int, eta=None, z=None,
                         w_out=None, stream=None):
    """The gate, then the TTT-Linear scan with its eta (include/ttt.h).
    Returns (z, w_out, eta)."""
    B, H, T, d = q.shape
    if tuple(x.shape[:2]) != (B, T):
        raise ValueError("x must be [B, T, dx] with the scan's B and T")
    _, _, _, dx, eta = _gate_common(x, theta_lr, H, eta)
    if z is None:
        z = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    if w_out is None:
        w_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    dev = _check_tensors(dict(q=q, k=k, v=v, x=x, theta_lr=theta_lr, w0=w0, eta=eta, z=z,
                              w_out=w_out))
    for name, t in (("w0", w0), ("z", z), ("w_out", w_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.shape != q.shape or v.shape != q.shape:
        raise TypeError("q, k, v must share one dtype and shape")
    per_batch = 1 if w0.dim() == 4 else 0
    if tuple(w0.shape) != ((B, H, d, d) if per_batch else (H, d, d)):
        raise ValueError(f"w0 has shape {tuple(w0.shape)}")
    if tuple(z.shape) != (B, H, T, d) or tuple(w_out.shape) != (B, H, d, d):
        raise ValueError("output shape mismatch")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_linear_gated_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(theta_lr), float(eta_base), dx, _ptr(w0),
            per_batch, B, H, T, d, int(b), _dtype_code(q), _ptr(eta), _ptr(z), _ptr(w_out),
            _stream(dev, stream)))
    return z, w_out, eta


def ttt_mlp_gated_fwd(q, k, v, x, theta_lr, eta_base: float, w1_0, w2_0, b: int, eta=None,
                      z=None, w1_out=None, w2_out=None, stream=None):
    """The gate, then the TTT-MLP scan with its eta (include/ttt.h).
    Returns (z, w1_out, w2_out, eta)."""
    B, H, T, d = q.shape
    hidden = w1_0.shape[-2]
    if tuple(x.shape[:2]) != (B, T):
        raise ValueError("x must be [B, T, dx] with the scan's B and T")
    _, _, _, dx, eta = _gate_common(x, theta_lr, H, eta)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    z = f32(B, H, T, d) if z is None else z
    w1_out = f32(B, H, hidden, d) if w1_out is None else w1_out
    w2_out = f32(B, H, d, hidden) if w2_out is None else w2_out
    dev = _check_tensors(dict(q=q, k=k, v=v, x=x, theta_lr=theta_lr, w1_0=w1_0, w2_0=w2_0,
                              eta=eta, z=z, w1_out=w1_out, w2_out=w2_out))
    for name, t in (("w1_0", w1_0), ("w2_0", w2_0), ("z", z), ("w1_out", w1_out),
                    ("w2_out", w2_out)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.shape != q.shape or v.shape != q.shape:
        raise TypeError("q, k, v must share one dtype and shape")
    per_batch = 1 if w1_0.dim() == 4 else 0
    lead = (B, H) if per_batch else (H,)
    if tuple(w1_0.shape) != (*lead, hidden, d) or tuple(w2_0.shape) != (*lead, d, hidden):
        raise ValueError("w1_0 / w2_0 shape mismatch")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_mlp_gated_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(theta_lr), float(eta_base), dx, _ptr(w1_0),
            _ptr(w2_0), per_batch, B, H, T, d, hidden, int(b), _dtype_code(q), _ptr(eta), _ptr(z),
            _ptr(w1_out), _ptr(w2_out), _stream(dev, stream)))
    return z, w1_out, w2_out, eta


def bench_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Streaming copy kernel used to calibrate hardware byte counters."""
    dev = _check_tensors(dict(src=src, dst=dst))
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst too small")
    with torch.cuda.device(dev):
        _lib.check(_lib.lib().ttt_bench_copy(_ptr(src), _ptr(dst), n, _stream(dev, stream)))
