"""Python entry points over libfa.so: fa_forward, fa_backward and an autograd.Function.

PyTorch supplies device memory and the current stream; the library does all the work.
Shapes follow "Systems and Parallelism" (CS336 field map, A2), problem flash_forward:
forward(Q, K, V, is_causal=False) returns O, and the only [batch, n_queries]-shaped tensor
saved for the backward is the logsumexp L.
"""
from __future__ import annotations

import functools
import math

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FA_DTYPE_F32, torch.bfloat16: _lib.FA_DTYPE_BF16}


def default_scale(d: int) -> float:
    """float32(1/sqrt(d)), the value passed to the kernels when no scale is given."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(name: str, t: torch.Tensor, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device} (a GPU device), got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")


def _raise(status: int, where: str):
    if status != _lib.FA_SUCCESS:
        raise _lib.FAError(status, where)


@functools.lru_cache(maxsize=256)
def _forward_ws_bytes(dtype: int, B: int, H: int, Nq: int, Nk: int, d: int, causal: int) -> int:
    return _lib.load().fa_forward_workspace_bytes(dtype, B, H, Nq, Nk, d, causal)


def forward_workspace_bytes(q: torch.Tensor, k: torch.Tensor, is_causal: bool) -> int:
    """Bytes of device workspace fa_forward can use for these shapes (0: none)."""
    B, H, Nq, d = q.shape
    return _forward_ws_bytes(_DTYPES[q.dtype], B, H, Nq, k.shape[2], d, int(bool(is_causal)))


def fa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool = False,
               scale: float | None = None, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """O, L = attention forward on [B, H, N, d] tensors (bf16 or fp32).

    `workspace` (uint8, on q's device) is allocated when not given and the shapes can use
    one (forward_workspace_bytes); pass a tensor to reuse it across calls."""
    lib = _lib.load()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2] if k.dim() == 4 else -1
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _check("q", q, (B, H, Nq, d), q.dtype, q.device)
    _check("k", k, (B, H, Nk, d), q.dtype, q.device)
    _check("v", v, (B, H, Nk, d), q.dtype, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check("out", out, (B, H, Nq, d), q.dtype, q.device)
    _check("lse", lse, (B, H, Nq), torch.float32, q.device)
    sc = default_scale(d) if scale is None else float(scale)
    if workspace is None:
        need = _forward_ws_bytes(_DTYPES[q.dtype], B, H, Nq, Nk, d, int(bool(is_causal)))
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (_DTYPES[q.dtype], B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
            int(bool(is_causal)), sc, out.data_ptr(), lse.data_ptr())
    if workspace is None:
        st = lib.fa_forward(*args, _stream_ptr(q))
        _raise(st, "fa_forward")
    else:
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
        st = lib.fa_forward_with_workspace(*args, workspace.data_ptr() if ws_bytes else None,
                                           ws_bytes, _stream_ptr(q))
        _raise(st, "fa_forward_with_workspace")
    return out, lse


def _backward_args(q, k, v, o, lse, do, dq, dk, dv, workspace):
    """Checked tensors and sizes shared by the backward entry points."""
    lib = _lib.load()
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for name, t, n in (("q", q, Nq), ("k", k, Nk), ("v", v, Nk), ("o", o, Nq), ("do", do, Nq)):
        _check(name, t, (B, H, n, d), dt, q.device)
    _check("lse", lse, (B, H, Nq), torch.float32, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, n in (("dq", dq, Nq), ("dk", dk, Nk), ("dv", dv, Nk)):
        _check(name, t, (B, H, n, d), dt, q.device)
    ws_bytes = lib.fa_backward_workspace_bytes(_DTYPES[dt], B, H, Nq, Nk, d)
    if workspace is not None:
        # bf16 needs two floats per query row; fa_backward_workspace_bytes may ask for more
        # (partial sums that let small causal grids use every CU), which is optional.
        need = B * H * Nq * 8 if dt == torch.bfloat16 else 0
        if (workspace.device != q.device or workspace.nbytes < need
                or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes "
                             f"({ws_bytes} for the fastest path) on {q.device}")
        ws, ws_bytes = workspace, workspace.nbytes
    else:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    return lib, (B, H, Nq, Nk, d), dq, dk, dv, ws, ws_bytes


def fa_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                lse: torch.Tensor, do: torch.Tensor, is_causal: bool = False,
                scale: float | None = None, dq: torch.Tensor | None = None,
                dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None):
    """dQ, dK, dV of the attention forward, from Q, K, V, O, L and dO.

    `workspace`, if given, is a device tensor of at least backward_workspace_bytes() bytes
    that the call may overwrite; otherwise one is allocated."""
    lib, (B, H, Nq, Nk, d), dq, dk, dv, ws, ws_bytes = _backward_args(
        q, k, v, o, lse, do, dq, dk, dv, workspace)
    sc = default_scale(d) if scale is None else float(scale)
    st = lib.fa_backward(_DTYPES[q.dtype], B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(),
                         v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                         int(bool(is_causal)), sc, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         ws.data_ptr() if ws is not None else None, ws_bytes, _stream_ptr(q))
    _raise(st, "fa_backward")
    return dq, dk, dv


def fa_backward_preprocess(o: torch.Tensor, lse: torch.Tensor, do: torch.Tensor,
                           workspace: torch.Tensor):
    """The backward's preprocessing step alone: per-row L log2(e) and -D into `workspace`."""
    lib = _lib.load()
    B, H, Nq, d = o.shape
    if o.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {o.dtype}")
    _check("o", o, (B, H, Nq, d), o.dtype, o.device)
    _check("do", do, (B, H, Nq, d), o.dtype, o.device)
    _check("lse", lse, (B, H, Nq), torch.float32, o.device)
    if workspace.device != o.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {o.device}")
    st = lib.fa_backward_preprocess(_DTYPES[o.dtype], B, H, Nq, d, o.data_ptr(), lse.data_ptr(),
                                    do.data_ptr(), workspace.data_ptr(), workspace.nbytes,
                                    _stream_ptr(o))
    _raise(st, "fa_backward_preprocess")


def fa_backward_main(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, do: torch.Tensor, is_causal: bool, scale: float | None,
                     workspace: torch.Tensor, dq: torch.Tensor | None = None,
                     dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Everything fa_backward does after fa_backward_preprocess filled `workspace`."""
    lib, (B, H, Nq, Nk, d), dq, dk, dv, ws, ws_bytes = _backward_args(
        q, k, v, o, lse, do, dq, dk, dv, workspace)
    sc = default_scale(d) if scale is None else float(scale)
    st = lib.fa_backward_main(_DTYPES[q.dtype], B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                              int(bool(is_causal)), sc, dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), ws.data_ptr(), ws_bytes, _stream_ptr(q))
    _raise(st, "fa_backward_main")
    return dq, dk, dv


def fa_backward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                        lse: torch.Tensor, do: torch.Tensor, is_causal: bool, scale: float | None,
                        dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor):
    """fa_backward with the library's static device workspace instead of one passed in, for
    callers that cannot allocate: the outputs must be given, and nothing is allocated."""
    lib = _lib.load()
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for name, t, n in (("q", q, Nq), ("k", k, Nk), ("v", v, Nk), ("o", o, Nq), ("do", do, Nq),
                       ("dq", dq, Nq), ("dk", dk, Nk), ("dv", dv, Nk)):
        _check(name, t, (B, H, n, d), dt, q.device)
    _check("lse", lse, (B, H, Nq), torch.float32, q.device)
    sc = default_scale(d) if scale is None else float(scale)
    st = lib.fa_backward_noalloc(_DTYPES[dt], B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(),
                                 v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                 int(bool(is_causal)), sc, dq.data_ptr(), dk.data_ptr(),
                                 dv.data_ptr(), _stream_ptr(q))
    _raise(st, "fa_backward_noalloc")
    return dq, dk, dv


def backward_workspace_bytes(q: torch.Tensor, k: torch.Tensor) -> int:
    """Bytes of workspace fa_backward needs for these query and key tensors."""
    B, H, Nq, d = q.shape
    return _lib.load().fa_backward_workspace_bytes(_DTYPES[q.dtype], B, H, Nq, k.shape[2], d)


def backward_atomic_workspace_bytes(q: torch.Tensor, k: torch.Tensor) -> int:
    """Bytes of workspace fa_backward_atomic needs for these query and key tensors."""
    B, H, Nq, d = q.shape
    return _lib.load().fa_backward_atomic_workspace_bytes(_DTYPES[q.dtype], B, H, Nq,
                                                          k.shape[2], d)


def fa_backward_atomic(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                       lse: torch.Tensor, do: torch.Tensor, is_causal: bool = False,
                       scale: float | None = None, dq: torch.Tensor | None = None,
                       dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None):
    """fa_backward with dQ accumulated by fp32 atomic additions (bf16 only). dK and dV are
    deterministic; dQ may differ between runs in its last bits (the order of the additions
    varies). `workspace`, if given, must hold backward_atomic_workspace_bytes() bytes."""
    if q.dtype != torch.bfloat16:
        raise TypeError("fa_backward_atomic supports bf16 inputs only")
    need = backward_atomic_workspace_bytes(q, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.nbytes < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    lib, (B, H, Nq, Nk, d), dq, dk, dv, ws, ws_bytes = _backward_args(
        q, k, v, o, lse, do, dq, dk, dv, workspace)
    sc = default_scale(d) if scale is None else float(scale)
    st = lib.fa_backward_atomic(_DTYPES[q.dtype], B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(),
                                v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                int(bool(is_causal)), sc, dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), ws.data_ptr(), ws_bytes, _stream_ptr(q))
    _raise(st, "fa_backward_atomic")
    return dq, dk, dv


def kernel_names(dtype: torch.dtype, B: int, H: int, Nq: int, Nk: int, d: int, is_causal: bool,
                 forward_workspace_bytes: int = 0, backward_workspace_bytes: int = 0):
    """(forward, backward) names of the attention kernels the library launches for these
    arguments and workspace sizes, from the library's own dispatch (fa_forward_kernel_name,
    fa_backward_kernel_name)."""
    lib = _lib.load()
    dt = _DTYPES[dtype]
    c = int(bool(is_causal))
    return (lib.fa_forward_kernel_name(dt, B, H, Nq, Nk, d, c, forward_workspace_bytes).decode(),
            lib.fa_backward_kernel_name(dt, B, H, Nq, Nk, d, c, backward_workspace_bytes).decode())


class FlashAttention(torch.autograd.Function):
    """Autograd wrapper: apply(Q, K, V, is_causal=False, scale=None) -> O."""

    @staticmethod
    def forward(ctx, q, k, v, is_causal=False, scale=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = fa_forward(q, k, v, is_causal, scale)
        ctx.save_for_backward(lse, q, k, v, o)
        ctx.is_causal = bool(is_causal)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        lse, q, k, v, o = ctx.saved_tensors
        dq, dk, dv = fa_backward(q, k, v, o, lse, do.contiguous(), ctx.is_causal, ctx.scale)
        return dq, dk, dv, None, None
