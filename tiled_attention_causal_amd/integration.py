"""Drop-in use of the flash kernels as a model's attention function.

"Systems and Parallelism" (CS336 field map, A2) plugs its FlashAttention-2 autograd function into
an existing Transformer by replacing the model module's attention function. Two pieces do that
here:

    from tiled_attention_causal_amd import integration
    with integration.patched(model_module, "scaled_dot_product_attention"):
        loss = model(x).sum()          # attention now runs on libfa.so, forward and backward
        loss.backward()

`scaled_dot_product_attention(q, k, v, mask=None, is_causal=False, scale=None)` keeps the usual
calling convention: q, k, v are [..., N, d] with any leading (batch, head) dimensions, and a mask,
if given, is a boolean keep-mask that must be the causal (lower-triangular) one. Anything the
kernels do not implement (another mask, an unsupported dtype or head dim, CPU tensors) raises
instead of silently computing attention some other way.
"""
from __future__ import annotations

import contextlib

import torch

from .ops import FlashAttention

_SUPPORTED_D = (16, 32, 64, 128)


def _is_causal_mask(mask: torch.Tensor, nq: int, nk: int) -> bool:
    """True when `mask` (boolean, keep = True, broadcastable to [..., nq, nk]) keeps exactly
    key j <= query i for every query row."""
    if mask.dtype != torch.bool or mask.shape[-2:] != (nq, nk):
        return False
    causal = torch.ones(nq, nk, dtype=torch.bool, device=mask.device).tril_()
    return bool(torch.equal(mask, causal.expand_as(mask)))


def scaled_dot_product_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                 mask: torch.Tensor | None = None, is_causal: bool = False,
                                 scale: float | None = None) -> torch.Tensor:
    """softmax(q k^T * scale [causal]) v on the flash kernels, differentiable in q, k and v."""
    if q.dim() < 2 or k.dim() != q.dim() or v.dim() != q.dim():
        raise ValueError("q, k and v must have the same rank, at least 2")
    nq, d = q.shape[-2:]
    nk = k.shape[-2]
    if mask is not None:
        if not _is_causal_mask(mask, nq, nk):
            raise NotImplementedError("only the causal keep-mask (lower-triangular) is supported")
        is_causal = True
    if d not in _SUPPORTED_D or v.shape[-1] != d or k.shape[-1] != d:
        raise NotImplementedError(f"head dim {d} (q), {k.shape[-1]} (k), {v.shape[-1]} (v): "
                                  f"the kernels take one of {_SUPPORTED_D} for all three")
    lead = q.shape[:-2]
    if k.shape[:-2] != lead or v.shape[:-2] != lead or v.shape[-2] != nk:
        raise ValueError("q, k and v must agree in their leading dimensions and k, v in N")
    bh = 1
    for s in lead:
        bh *= s
    o = FlashAttention.apply(q.reshape(1, bh, nq, d), k.reshape(1, bh, nk, d),
                             v.reshape(1, bh, nk, d), bool(is_causal), scale)
    return o.reshape(*lead, nq, d)


@contextlib.contextmanager
def patched(module, name: str = "scaled_dot_product_attention", fn=None):
    """Within the block, `module.<name>` is the flash attention function (or `fn`); the
    original attribute is restored on exit, also when the block raises."""
    if not hasattr(module, name):
        raise AttributeError(f"{module!r} has no attribute {name!r} to replace")
    old = getattr(module, name)
    setattr(module, name, scaled_dot_product_attention if fn is None else fn)
    try:
        yield
    finally:
        setattr(module, name, old)
