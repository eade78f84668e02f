"""ctypes loader for libttt.so (the C ABI declared in include/ttt.h and
include/ttt_tuning.h).  There is no fallback: if the library is missing the
import of any entry point raises."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt.so")

STATUS = {
    0: "TTT_OK", 1: "TTT_ERR_NULL", 2: "TTT_ERR_SHAPE", 3: "TTT_ERR_DTYPE",
    4: "TTT_ERR_UNSUPPORTED", 5: "TTT_ERR_ALIAS", 6: "TTT_ERR_HIP", 7: "TTT_ERR_ALIGN",
    8: "TTT_ERR_VALUE",
}
TTT_F32, TTT_BF16 = 0, 1

# name -> (restype, argtypes)
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "ttt_linear_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                              _vp, _vp, _vp]),
    "ttt_linear_fwd_tuned": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _vp, _vp, _vp, _i32]),
    "ttt_linear_fwd_ring_depth": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _vp, _vp, _vp, _i32, _i32]),
    "ttt_linear_fwd_chunked": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _vp, _vp, _vp, _i32, _i32]),
    "ttt_linear_fwd_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "ttt_linear_ln_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, ctypes.c_float, _i32,
                                 _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "ttt_mlp_ln_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, ctypes.c_float, _i32,
                              _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "ttt_linear_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                               _vp, _vp]),
    "ttt_linear_ln_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                  _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "ttt_linear_fwd_ckpt": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _vp, _vp, _vp, _vp]),
    "ttt_linear_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp]),
    "ttt_linear_bwd_chunked": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32]),
    "ttt_lr_gate": (_i32, [_vp, _i32, _vp, ctypes.c_float, _i32, _i32, _i32, _i32, _vp, _vp]),
    "ttt_lr_gate_bwd": (_i32, [_vp, _i32, _vp, ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _i32,
                               _vp, _vp, _vp]),
    "ttt_lr_gate_tuned": (_i32, [_vp, _i32, _vp, ctypes.c_float, _i32, _i32, _i32, _i32, _vp, _vp,
                                 _i32]),
    "ttt_linear_gated_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _i32, _vp, _i32,
                                    _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "ttt_mlp_gated_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _i32, _vp, _vp, _i32,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _vp]),
    "ttt_mlp_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                            _i32, _i32, _vp, _vp]),
    "ttt_mlp_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           _i32, _vp, _vp, _vp, _vp]),
    "ttt_linear_ln_fwd_ckpt": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, ctypes.c_float,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "ttt_linear_ln_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp]),
    "ttt_mlp_fwd_ckpt": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ttt_mlp_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ttt_status_str": (ctypes.c_char_p, [_i32]),
    "ttt_last_error": (ctypes.c_char_p, []),
    "ttt_abi_version": (_i32, []),
    "ttt_bench_copy": (_i32, [_vp, _vp, _sz, _vp]),
}


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is not built; run `python -m test_rnn_layers_head_amd.build` "
                    "(the TTT scan has no non-HIP implementation)")
            cdll = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(cdll, name)
                fn.restype, fn.argtypes = res, args
            _lib = cdll
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise TTTError(status, lib().ttt_last_error().decode(errors="replace"))
