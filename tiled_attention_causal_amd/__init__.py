"""FlashAttention-2 style causal attention for MI355X (gfx950): HIP kernels behind a C ABI.

    from tiled_attention_causal_amd import fa_forward, fa_backward, FlashAttention
"""
from ._lib import FAError, LIB_PATH, load  # noqa: F401
from .ops import (FlashAttention, backward_atomic_workspace_bytes,  # noqa: F401
                  backward_workspace_bytes, default_scale, fa_backward, fa_backward_atomic,
                  fa_backward_main, fa_backward_noalloc, fa_backward_preprocess, fa_forward,
                  forward_workspace_bytes, kernel_names)

__all__ = ["fa_forward", "fa_backward", "fa_backward_preprocess", "fa_backward_main",
           "fa_backward_atomic", "fa_backward_noalloc", "forward_workspace_bytes",
           "backward_workspace_bytes", "backward_atomic_workspace_bytes", "kernel_names", "FlashAttention",
           "default_scale", "FAError", "load", "LIB_PATH"]
