"""MI355X-native TTT forward scan (TTT-Linear / TTT-MLP, mini-batch dual form).

The scan runs in hand-written gfx950 HIP kernels behind the C ABI of
libttt.so (include/ttt.h); this package is its thin Python binding.
"""
from .api import (bench_copy, ttt_linear_bwd, ttt_linear_fwd, ttt_linear_fwd_ckpt,  # noqa: F401
                  ttt_linear_fwd_plan,
                  ttt_linear_gated_fwd, ttt_linear_ln_bwd, ttt_linear_ln_fwd,
                  ttt_linear_ln_fwd_ckpt, ttt_linear_ln_step, ttt_linear_step,
                  ttt_lr_gate, ttt_lr_gate_bwd, ttt_mlp_bwd, ttt_mlp_fwd, ttt_mlp_fwd_ckpt,
                  ttt_mlp_ln_fwd,
                  ttt_mlp_gated_fwd, ttt_mlp_step)
from ._lib import TTTError  # noqa: F401
