"""MI355X (gfx950) DeepSeekMoE layer forward with aux-loss-free load balancing.

The computation runs in libmoe.so (hand-written HIP kernels behind a C ABI declared
in include/moe.h); this package holds the ctypes binding (`_lib`), a buffer-owning
layer object (`layer.MoELayer`) and the build script (`build`).
"""
from ._lib import (MoeError, moe_bias_update, moe_combine, moe_expert_ffn, moe_permute,  # noqa: F401
                   moe_quantize_weights_fp8, moe_route, moe_workspace_bytes, problem)

__all__ = ["MoeError", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_bias_update", "moe_quantize_weights_fp8", "moe_workspace_bytes", "problem"]
