"""The C ABI of libttt.so, host side only (no GPU needed): the library loads,
exports every function that include/*.h declares with the signature the
binding uses, and rejects bad arguments before anything reaches the GPU.

Every call below returns from argument validation (or from the empty-work
shortcut) before the first HIP runtime call; the pointers passed are never
dereferenced.
"""
import ctypes
import glob
import os
import re

import pytest

from test_rnn_layers_head_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^\s*(?:const\s+)?[A-Za-z_]\w*\s*\*?\s*(ttt_\w+)\s*\(", re.M)


def declared():
    names = {}
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        for m in DECL.finditer(open(h).read()):
            names[m.group(1)] = os.path.basename(h)
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from test_rnn_layers_head_amd import build
        build.build()
    return _lib.lib()


def header_value(name):
    text = open(os.path.join(ROOT, "include", "ttt.h")).read()
    return int(re.search(rf"#define {name} (\d+)", text).group(1))


def test_headers_declare_the_entry_points():
    names = declared()
    for fn in ("ttt_linear_fwd", "ttt_linear_ln_fwd", "ttt_mlp_fwd", "ttt_linear_fwd_tuned",
               "ttt_bench_copy", "ttt_status_str", "ttt_last_error", "ttt_abi_version"):
        assert fn in names, fn


def test_every_declared_symbol_is_exported_and_bound(lib):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name, header in declared().items():
        assert hasattr(raw, name), f"{name} ({header}) is not exported"
        assert name in _lib.SIGNATURES, f"{name} ({header}) has no ctypes signature"
    assert set(_lib.SIGNATURES) <= set(declared())


def test_version_and_status_strings(lib):
    assert lib.ttt_abi_version() == header_value("TTT_ABI_VERSION")
    for code, name in _lib.STATUS.items():
        assert lib.ttt_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.ttt_status_str(99)


# fake device addresses: 16-byte aligned, disjoint, never dereferenced
A = [0x10000000 * (i + 1) for i in range(14)]
P, M = 0x20000, 0x30000  # unaligned / overlapping variants


def linear(lib, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], eta=A[3], w0=A[4], per_batch=0, B=1, H=1, T=16, d=64,
                b=16, dt=_lib.TTT_BF16, z=A[5], w=A[6])
    args.update(kw)
    return lib.ttt_linear_fwd(args["q"], args["k"], args["v"], args["eta"], args["w0"],
                              args["per_batch"], args["B"], args["H"], args["T"], args["d"],
                              args["b"], args["dt"], args["z"], args["w"], None)


def linear_chunked(lib, rows=0, chunks=2, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], eta=A[3], w0=A[4], per_batch=0, B=1, H=1, T=1024, d=64,
                b=16, dt=_lib.TTT_BF16, z=A[5], w=A[6])
    args.update(kw)
    return lib.ttt_linear_fwd_chunked(args["q"], args["k"], args["v"], args["eta"], args["w0"],
                                      args["per_batch"], args["B"], args["H"], args["T"],
                                      args["d"], args["b"], args["dt"], args["z"], args["w"], None,
                                      rows, chunks)


@pytest.mark.parametrize("kw,expect", [
    (dict(chunks=-1), "TTT_ERR_UNSUPPORTED"),
    (dict(chunks=3), "TTT_ERR_UNSUPPORTED"),             # 1024 not a multiple of 3
    (dict(chunks=8), "TTT_ERR_UNSUPPORTED"),             # 128-token chunks (< 192)
    (dict(chunks=2, T=1000), "TTT_ERR_UNSUPPORTED"),     # 500-token chunks, not 16 | 500
    (dict(chunks=2, dt=_lib.TTT_F32), "TTT_ERR_UNSUPPORTED"),
    (dict(chunks=2, b=4), "TTT_ERR_UNSUPPORTED"),
    (dict(chunks=2, rows=24), "TTT_ERR_UNSUPPORTED"),
    (dict(chunks=2, z=A[0]), "TTT_ERR_ALIAS"),
    (dict(chunks=2, B=0), "TTT_OK"),                      # empty work: nothing launched
])
def test_linear_chunked_argument_checks(lib, kw, expect):
    assert linear_chunked(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_fwd_chunked:")


@pytest.mark.parametrize("depth,b,dt,kw,expect", [
    (2, 16, _lib.TTT_BF16, {}, "TTT_ERR_UNSUPPORTED"),
    (-1, 16, _lib.TTT_BF16, {}, "TTT_ERR_UNSUPPORTED"),
    (1, 8, _lib.TTT_BF16, {}, "TTT_ERR_UNSUPPORTED"),
    (1, 16, _lib.TTT_F32, {}, "TTT_ERR_UNSUPPORTED"),
    (1, 16, _lib.TTT_BF16, dict(z=A[0]), "TTT_ERR_ALIAS"),
    (1, 16, _lib.TTT_BF16, dict(B=0), "TTT_OK"),
])
def test_linear_ring_depth_argument_checks(lib, depth, b, dt, kw, expect):
    args = dict(q=A[0], k=A[1], v=A[2], eta=A[3], w0=A[4], B=1, H=1, T=64, z=A[5], w=A[6])
    args.update(kw)
    r = lib.ttt_linear_fwd_ring_depth(args["q"], args["k"], args["v"], args["eta"], args["w0"], 0,
                                      args["B"], args["H"], args["T"], 64, b, dt, args["z"],
                                      args["w"], None, 0, depth)
    assert r == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_fwd_ring_depth:")


@pytest.mark.parametrize("B,H,T,b,dt,want", [
    (4, 32, 8192, 16, _lib.TTT_BF16, (32, 1)),      # the 1.3B workload: one pass
    (1, 32, 32768, 16, _lib.TTT_BF16, (64, 8)),     # long context: 8 chunks of 4096
    (1, 2, 8192, 16, _lib.TTT_BF16, (16, 8)),       # chunks of at least 1024 tokens
    (1, 32, 32768, 4, _lib.TTT_BF16, (16, 1)),      # chunking needs b = 16
    (1, 32, 32768, 16, _lib.TTT_F32, (16, 1)),      # and bf16 inputs
    (16, 16, 8192, 16, _lib.TTT_BF16, (64, 1)),     # 256 units
])
def test_linear_fwd_plan(lib, B, H, T, b, dt, want):
    import ctypes
    rows, chunks = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert lib.ttt_linear_fwd_plan(B, H, T, b, dt, ctypes.addressof(rows),
                                   ctypes.addressof(chunks)) == 0
    assert (rows.value, chunks.value) == want


def test_linear_fwd_plan_errors(lib):
    import ctypes
    r, c = ctypes.c_int32(0), ctypes.c_int32(0)
    ra, ca = ctypes.addressof(r), ctypes.addressof(c)
    assert lib.ttt_linear_fwd_plan(1, 1, 16, 16, _lib.TTT_BF16, None, ca) == status("TTT_ERR_NULL")
    assert lib.ttt_linear_fwd_plan(-1, 1, 16, 16, _lib.TTT_BF16, ra, ca) == status("TTT_ERR_SHAPE")
    assert lib.ttt_linear_fwd_plan(1, 1, 16, 0, _lib.TTT_BF16, ra, ca) == status("TTT_ERR_SHAPE")
    assert lib.ttt_linear_fwd_plan(1, 1, 16, 16, 7, ra, ca) == status("TTT_ERR_DTYPE")
    assert lib.ttt_last_error().startswith(b"ttt_linear_fwd_plan:")


def linear_ln(lib, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], eta=A[3], w0=A[4], per_batch=0, gamma=A[7], beta=A[8],
                eps=1e-5, B=1, H=1, T=16, d=64, b=16, dt=_lib.TTT_BF16, z=A[5], w=A[6])
    args.update(kw)
    return lib.ttt_linear_ln_fwd(args["q"], args["k"], args["v"], args["eta"], args["w0"],
                                 args["per_batch"], args["gamma"], args["beta"], args["eps"],
                                 args["B"], args["H"], args["T"], args["d"], args["b"],
                                 args["dt"], args["z"], args["w"], None)


def status(code):
    return {v: k for k, v in _lib.STATUS.items()}[code]


@pytest.mark.parametrize("kw,expect", [
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),
    (dict(b=24), "TTT_ERR_UNSUPPORTED"),
    (dict(b=0), "TTT_ERR_UNSUPPORTED"),
    (dict(B=-1), "TTT_ERR_SHAPE"),
    (dict(per_batch=2), "TTT_ERR_SHAPE"),
    (dict(dt=7), "TTT_ERR_DTYPE"),
    (dict(q=None), "TTT_ERR_NULL"),
    (dict(eta=A[3] + 4), "TTT_ERR_ALIGN"),
    (dict(z=A[1]), "TTT_ERR_ALIAS"),
    (dict(w=A[4]), "TTT_ERR_ALIAS"),            # in place needs w0_per_batch = 1
    (dict(B=1 << 20, H=1 << 10, T=1 << 10), "TTT_ERR_SHAPE"),
    (dict(B=1, H=1, T=1 << 24), "TTT_ERR_SHAPE"),   # one unit's z past 32-bit offsets
    (dict(B=0), "TTT_OK"),                      # empty work: nothing launched
    (dict(H=0), "TTT_OK"),
])
def test_linear_argument_checks(lib, kw, expect):
    assert linear(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_fwd:")


@pytest.mark.parametrize("kw,expect", [
    (dict(eps=0.0), "TTT_ERR_VALUE"),
    (dict(eps=-1.0), "TTT_ERR_VALUE"),
    (dict(eps=float("nan")), "TTT_ERR_VALUE"),
    (dict(eps=float("inf")), "TTT_ERR_VALUE"),
    (dict(b=24), "TTT_ERR_UNSUPPORTED"),
    (dict(b=3), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=6), "TTT_ERR_DTYPE"),
    (dict(gamma=None), "TTT_ERR_NULL"),
    (dict(beta=A[8] + 8), "TTT_ERR_ALIGN"),
    (dict(z=A[7]), "TTT_ERR_ALIAS"),
    (dict(B=0), "TTT_OK"),
])
def test_linear_ln_argument_checks(lib, kw, expect):
    assert linear_ln(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_ln_fwd:")


def mlp_ln(lib, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], eta=A[3], w1=A[4], w2=A[9], per_batch=0, gamma=A[7],
                beta=A[8], eps=1e-5, B=1, H=1, T=16, d=64, hidden=256, b=16, dt=_lib.TTT_BF16,
                z=A[5], w1o=A[6], w2o=A[10])
    args.update(kw)
    return lib.ttt_mlp_ln_fwd(args["q"], args["k"], args["v"], args["eta"], args["w1"],
                              args["w2"], args["per_batch"], args["gamma"], args["beta"],
                              args["eps"], args["B"], args["H"], args["T"], args["d"],
                              args["hidden"], args["b"], args["dt"], args["z"], args["w1o"],
                              args["w2o"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(eps=0.0), "TTT_ERR_VALUE"),
    (dict(eps=float("nan")), "TTT_ERR_VALUE"),
    (dict(b=24), "TTT_ERR_UNSUPPORTED"),
    (dict(hidden=128), "TTT_ERR_UNSUPPORTED"),
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=6), "TTT_ERR_DTYPE"),
    (dict(gamma=None), "TTT_ERR_NULL"),
    (dict(w2=None), "TTT_ERR_NULL"),
    (dict(beta=A[8] + 8), "TTT_ERR_ALIGN"),
    (dict(z=A[7]), "TTT_ERR_ALIAS"),
    (dict(w1o=A[9]), "TTT_ERR_ALIAS"),
    (dict(T=1 << 24), "TTT_ERR_SHAPE"),
    (dict(B=0), "TTT_OK"),
])
def test_mlp_ln_argument_checks(lib, kw, expect):
    assert mlp_ln(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_mlp_ln_fwd:")


def test_mlp_argument_checks(lib):
    f = lambda **kw: lib.ttt_mlp_fwd(A[0], A[1], A[2], A[3], A[4], A[9], 0, 1, 1, 16, 64,
                                     kw.get("hidden", 256), kw.get("b", 16),
                                     kw.get("dt", _lib.TTT_BF16), A[5], A[6], A[10], None)
    assert f(hidden=128) == status("TTT_ERR_UNSUPPORTED")
    assert f(b=24) == status("TTT_ERR_UNSUPPORTED")  # neither b | 16 nor 16 | b
    assert f(b=3) == status("TTT_ERR_UNSUPPORTED")
    assert f(dt=7) == status("TTT_ERR_DTYPE")
    assert f(hidden=-1) == status("TTT_ERR_SHAPE")


def gate(lib, **kw):
    args = dict(x=A[0], dt=_lib.TTT_BF16, theta=A[1], eta_base=0.1, B=1, T=16, H=2, dx=64,
                eta=A[2])
    args.update(kw)
    return lib.ttt_lr_gate(args["x"], args["dt"], args["theta"], args["eta_base"], args["B"],
                           args["T"], args["H"], args["dx"], args["eta"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dx=48), "TTT_ERR_UNSUPPORTED"),
    (dict(dx=0), "TTT_ERR_UNSUPPORTED"),
    (dict(dx=-32), "TTT_ERR_SHAPE"),
    (dict(T=-1), "TTT_ERR_SHAPE"),
    (dict(dt=_lib.TTT_F32), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=7), "TTT_ERR_DTYPE"),
    (dict(eta_base=float("nan")), "TTT_ERR_VALUE"),
    (dict(eta_base=float("-inf")), "TTT_ERR_VALUE"),
    (dict(x=None), "TTT_ERR_NULL"),
    (dict(eta=None), "TTT_ERR_NULL"),
    (dict(theta=A[1] + 4), "TTT_ERR_ALIGN"),
    (dict(eta=A[0] + 64), "TTT_ERR_ALIAS"),     # inside x
    (dict(eta=A[1]), "TTT_ERR_ALIAS"),          # theta_lr
    (dict(B=1 << 16, T=1 << 12, H=1 << 4), "TTT_ERR_SHAPE"),
    (dict(B=0), "TTT_OK"),
    (dict(H=0), "TTT_OK"),
])
def test_lr_gate_argument_checks(lib, kw, expect):
    assert gate(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_lr_gate:")


def test_lr_gate_tuned_rejects_launch_shapes(lib):
    f = lambda tpw: lib.ttt_lr_gate_tuned(A[0], _lib.TTT_BF16, A[1], 0.1, 1, 16, 2, 64, A[2],
                                          None, tpw)
    assert f(48) == status("TTT_ERR_UNSUPPORTED")
    assert f(16) == status("TTT_ERR_UNSUPPORTED")


def gated_linear(lib, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], x=A[7], theta=A[8], eta_base=1.0, dx=64, w0=A[4],
                per_batch=0, B=1, H=1, T=16, d=64, b=16, dt=_lib.TTT_BF16, eta=A[3], z=A[5],
                w=A[6])
    args.update(kw)
    a = args
    return lib.ttt_linear_gated_fwd(a["q"], a["k"], a["v"], a["x"], a["theta"], a["eta_base"],
                                    a["dx"], a["w0"], a["per_batch"], a["B"], a["H"], a["T"],
                                    a["d"], a["b"], a["dt"], a["eta"], a["z"], a["w"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dx=40), "TTT_ERR_UNSUPPORTED"),       # the gate's checks
    (dict(theta=None), "TTT_ERR_NULL"),
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),        # the scan's checks, before any launch
    (dict(z=A[1]), "TTT_ERR_ALIAS"),
    (dict(eta=A[0]), "TTT_ERR_ALIAS"),          # eta over q
    (dict(eta=A[4]), "TTT_ERR_ALIAS"),          # eta over w0
    (dict(z=A[7]), "TTT_ERR_ALIAS"),            # z over x
    (dict(w=A[8]), "TTT_ERR_ALIAS"),            # w_out over theta_lr
    (dict(B=0), "TTT_OK"),
])
def test_linear_gated_argument_checks(lib, kw, expect):
    assert gated_linear(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_gated_fwd:")


def test_mlp_gated_argument_checks(lib):
    f = lambda **kw: lib.ttt_mlp_gated_fwd(A[0], A[1], A[2], A[7], A[8], 0.1, kw.get("dx", 64),
                                           A[4], A[9], 0, 1, 1, 16, 64, kw.get("hidden", 256),
                                           16, _lib.TTT_BF16, kw.get("eta", A[3]), A[5], A[6],
                                           A[10], None)
    assert f(hidden=128) == status("TTT_ERR_UNSUPPORTED")
    assert f(dx=33) == status("TTT_ERR_UNSUPPORTED")
    assert f(eta=A[9]) == status("TTT_ERR_ALIAS")
    assert lib.ttt_last_error().startswith(b"ttt_mlp_gated_fwd:")


def bwd(lib, **kw):
    args = dict(q=A[0], k=A[1], v=A[2], eta=A[3], ck=A[4], B=1, H=2, T=37, d=64, b=16,
                dt=_lib.TTT_BF16, dz=A[5], dwT=None, dq=A[6], dk=A[7], dv=A[8], deta=A[9],
                dw0=A[10])
    args.update(kw)
    a = args
    return lib.ttt_linear_bwd(a["q"], a["k"], a["v"], a["eta"], a["ck"], a["B"], a["H"], a["T"],
                              a["d"], a["b"], a["dt"], a["dz"], a["dwT"], a["dq"], a["dk"],
                              a["dv"], a["deta"], a["dw0"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(b=24), "TTT_ERR_UNSUPPORTED"),        # neither b | 16 nor 16 | b
    (dict(b=0), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=9), "TTT_ERR_DTYPE"),
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),
    (dict(T=-1), "TTT_ERR_SHAPE"),
    (dict(ck=None), "TTT_ERR_NULL"),
    (dict(dz=A[5] + 8), "TTT_ERR_ALIGN"),
    (dict(dq=A[4]), "TTT_ERR_ALIAS"),          # an output over the checkpoints
    (dict(dw0=A[6] + 256), "TTT_ERR_ALIAS"),    # two outputs
    (dict(dv=A[11], dwT=A[11] + 64), "TTT_ERR_ALIAS"),
    (dict(B=1, H=1, T=1 << 24), "TTT_ERR_SHAPE"),   # T x 64 fp32 outputs past 32-bit offsets
    (dict(B=0), "TTT_OK"),
])
def test_linear_bwd_argument_checks(lib, kw, expect):
    assert bwd(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_bwd:")


def test_linear_fwd_ckpt_argument_checks(lib):
    f = lambda **kw: lib.ttt_linear_fwd_ckpt(A[0], A[1], A[2], A[3], A[4], 0, 1, 1, 16, 64,
                                             kw.get("b", 16), kw.get("dt", _lib.TTT_BF16), A[5],
                                             A[6], kw.get("ck", A[7]), None)
    assert f(b=24) == status("TTT_ERR_UNSUPPORTED")
    assert f(dt=9) == status("TTT_ERR_DTYPE")
    assert f(ck=None) == status("TTT_ERR_NULL")
    assert f(ck=A[0]) == status("TTT_ERR_ALIAS")


def gate_bwd(lib, **kw):
    args = dict(x=A[0], dt=_lib.TTT_BF16, theta=A[1], eta_base=0.1, eta=A[2], deta=A[3], B=1,
                T=16, H=2, dx=64, dth=A[4], dxo=A[5])
    args.update(kw)
    a = args
    return lib.ttt_lr_gate_bwd(a["x"], a["dt"], a["theta"], a["eta_base"], a["eta"], a["deta"],
                               a["B"], a["T"], a["H"], a["dx"], a["dth"], a["dxo"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dx=48), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=_lib.TTT_F32), "TTT_ERR_UNSUPPORTED"),
    (dict(T=-1), "TTT_ERR_SHAPE"),
    (dict(T=1 << 20, H=1 << 10), "TTT_ERR_SHAPE"),   # B*T*H = 2^30
    (dict(eta_base=float("nan")), "TTT_ERR_VALUE"),
    (dict(deta=None), "TTT_ERR_NULL"),
    (dict(eta=A[2] + 4), "TTT_ERR_ALIGN"),
    (dict(dxo=A[0]), "TTT_ERR_ALIAS"),          # dx over x
    (dict(dth=A[3]), "TTT_ERR_ALIAS"),          # dtheta over deta
    (dict(dth=A[5] + 256), "TTT_ERR_ALIAS"),    # the two outputs
])
def test_lr_gate_bwd_argument_checks(lib, kw, expect):
    assert gate_bwd(lib, **kw) == status(expect), lib.ttt_last_error()
    assert lib.ttt_last_error().startswith(b"ttt_lr_gate_bwd:")


def bwd_chunked(lib, chunks, **kw):
    a = dict(q=A[0], k=A[1], v=A[2], eta=A[3], ck=A[4], B=1, H=2, T=768, d=64, b=16,
             dt=_lib.TTT_BF16, dz=A[5], dwT=None, dq=A[6], dk=A[7], dv=A[8], deta=A[9], dw0=A[10])
    a.update(kw)
    return lib.ttt_linear_bwd_chunked(a["q"], a["k"], a["v"], a["eta"], a["ck"], a["B"], a["H"],
                                      a["T"], a["d"], a["b"], a["dt"], a["dz"], a["dwT"], a["dq"],
                                      a["dk"], a["dv"], a["deta"], a["dw0"], None, chunks)


@pytest.mark.parametrize("chunks,kw,expect", [
    (-1, {}, "TTT_ERR_UNSUPPORTED"),
    (5, {}, "TTT_ERR_UNSUPPORTED"),                 # 768 not a multiple of 5
    (8, {}, "TTT_ERR_UNSUPPORTED"),                 # 96-token chunks (< 192)
    (2, dict(T=808), "TTT_ERR_UNSUPPORTED"),        # 404-token chunks, not 16 | 404
    (2, dict(b=4), "TTT_ERR_UNSUPPORTED"),
    (2, dict(dq=A[4]), "TTT_ERR_ALIAS"),
    (2, dict(dz=None), "TTT_ERR_NULL"),
    (2, dict(B=1, H=1, T=1 << 24), "TTT_ERR_SHAPE"),
    (4, dict(B=0), "TTT_OK"),                       # empty work: nothing launched
])
def test_linear_bwd_chunked_argument_checks(lib, chunks, kw, expect):
    assert bwd_chunked(lib, chunks, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_bwd_chunked:")


def mlp_bwd(lib, **kw):
    a = dict(q=A[0], k=A[1], v=A[2], eta=A[3], c1=A[4], c2=A[5], B=1, H=2, T=37, d=64, hidden=256,
             b=16, dt=_lib.TTT_BF16, dz=A[6], d1=None, d2=None, dq=A[7], dk=A[8], dv=A[9],
             deta=A[10], dw1=A[11], dw2=A[12])
    a.update(kw)
    return lib.ttt_mlp_bwd(a["q"], a["k"], a["v"], a["eta"], a["c1"], a["c2"], a["B"], a["H"],
                           a["T"], a["d"], a["hidden"], a["b"], a["dt"], a["dz"], a["d1"], a["d2"],
                           a["dq"], a["dk"], a["dv"], a["deta"], a["dw1"], a["dw2"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(b=24), "TTT_ERR_UNSUPPORTED"),
    (dict(hidden=128), "TTT_ERR_UNSUPPORTED"),
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=5), "TTT_ERR_DTYPE"),
    (dict(T=-1), "TTT_ERR_SHAPE"),
    (dict(B=1, H=1, T=1 << 24), "TTT_ERR_SHAPE"),
    (dict(c2=None), "TTT_ERR_NULL"),
    (dict(dz=A[6] + 4), "TTT_ERR_ALIGN"),
    (dict(dq=A[4]), "TTT_ERR_ALIAS"),            # an output over the checkpoints
    (dict(dw2=A[11] + 1024), "TTT_ERR_ALIAS"),   # two outputs
    (dict(B=0), "TTT_OK"),
])
def test_mlp_bwd_argument_checks(lib, kw, expect):
    assert mlp_bwd(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_mlp_bwd:")


def test_mlp_fwd_ckpt_argument_checks(lib):
    f = lambda **kw: lib.ttt_mlp_fwd_ckpt(A[0], A[1], A[2], A[3], A[4], A[9], 0, 1, 1, 16, 64,
                                          256, kw.get("b", 16), _lib.TTT_BF16, A[5], A[6], A[10],
                                          kw.get("c1", A[11]), kw.get("c2", A[12]), None)
    assert f(c1=None) == status("TTT_ERR_NULL")
    assert f(c2=A[0]) == status("TTT_ERR_ALIAS")     # checkpoints over q
    assert f(b=24) == status("TTT_ERR_UNSUPPORTED")


def ln_bwd(lib, **kw):
    a = dict(q=A[0], k=A[1], v=A[2], eta=A[3], ck=A[4], gamma=A[5], beta=A[6], eps=1e-5, B=1, H=2,
             T=37, d=64, b=16, dt=_lib.TTT_BF16, dz=A[7], dwT=None, dq=A[8], dk=A[9], dv=A[10],
             deta=A[11], dw0=A[12], dg=A[13], db=A[13] + 4096)
    a.update(kw)
    return lib.ttt_linear_ln_bwd(a["q"], a["k"], a["v"], a["eta"], a["ck"], a["gamma"], a["beta"],
                                 a["eps"], a["B"], a["H"], a["T"], a["d"], a["b"], a["dt"], a["dz"],
                                 a["dwT"], a["dq"], a["dk"], a["dv"], a["deta"], a["dw0"], a["dg"],
                                 a["db"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(b=24), "TTT_ERR_UNSUPPORTED"),
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),
    (dict(dt=4), "TTT_ERR_DTYPE"),
    (dict(eps=0.0), "TTT_ERR_VALUE"),
    (dict(T=-1), "TTT_ERR_SHAPE"),
    (dict(B=1, H=1, T=1 << 24), "TTT_ERR_SHAPE"),
    (dict(ck=None), "TTT_ERR_NULL"),
    (dict(gamma=None, T=0), "TTT_ERR_NULL"),     # gamma, beta needed even without tokens
    (dict(dz=A[7] + 4), "TTT_ERR_ALIGN"),
    (dict(dq=A[4]), "TTT_ERR_ALIAS"),            # an output over the checkpoints
    (dict(db=A[13] + 256), "TTT_ERR_ALIAS"),     # dgamma and dbeta overlap
    (dict(B=0), "TTT_OK"),
])
def test_linear_ln_bwd_argument_checks(lib, kw, expect):
    assert ln_bwd(lib, **kw) == status(expect), lib.ttt_last_error()
    if expect != "TTT_OK":
        assert lib.ttt_last_error().startswith(b"ttt_linear_ln_bwd:")


def test_linear_ln_fwd_ckpt_argument_checks(lib):
    f = lambda **kw: lib.ttt_linear_ln_fwd_ckpt(A[0], A[1], A[2], A[3], A[4], 0, A[7], A[8], 1e-5,
                                                1, 1, 16, 64, kw.get("b", 16), _lib.TTT_BF16, A[5],
                                                A[6], kw.get("ck", A[9]), None)
    assert f(ck=None) == status("TTT_ERR_NULL")
    assert f(ck=A[0]) == status("TTT_ERR_ALIAS")
    assert f(b=24) == status("TTT_ERR_UNSUPPORTED")
    assert lib.ttt_last_error().startswith(b"ttt_linear_ln_fwd_ckpt:")
