"""Python binding of libjattn.so: argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the computation runs in the
library's kernels. Layouts: q, k, v, out, dout, dq, dk, dv are bf16 [B, L, H, D] contiguous;
gains fp32 [2, D] (row 0 for Q, row 1 for K); valid_len int32 [B] (keys per sequence) or None;
lse fp32 [B, H, L] (natural-log row log-sum-exp).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib

__all__ = ["forward", "backward", "workspace_bytes", "fwd_workspace_bytes", "JointAttention", "joint_attention"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device} (contiguous={t.is_contiguous()})")


def _check_common(q, k, v, gains, valid_len):
    if q.dim() != 4:
        raise ValueError("q must be [B, L, H, D]")
    B, L, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, (B, L, H, D), dev)
    _check_tensor("gains", gains, torch.float32, (2, D), dev)
    if valid_len is not None:
        _check_tensor("valid_len", valid_len, torch.int32, (B,), dev)
    return B, L, H, D


def forward(q, k, v, gains, valid_len=None, scale: Optional[float] = None, eps: float = 1e-6,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, return_workspace: bool = False):
    """Joint attention forward. Returns (out bf16 [B, L, H, D], lse fp32 [B, H, L]), plus the forward
    workspace (the normalised key rows, reusable by `backward`) if return_workspace."""
    B, L, H, D = _check_common(q, k, v, gains, valid_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, (B, L, H, D), q.device)
    _check_tensor("lse", lse, torch.float32, (B, H, L), q.device)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(int(lib.jattn_fwd_workspace_bytes(B, L, H, D)), 1), dtype=torch.uint8,
                                device=q.device)
    st = lib.jattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(valid_len), B, L, H, D,
                       ctypes.c_float(scale), ctypes.c_float(eps), _ptr(out), _ptr(lse), _ptr(workspace),
                       workspace.numel(), _stream(q))
    _lib.check("jattn_fwd", st)
    return (out, lse, workspace) if return_workspace else (out, lse)


def workspace_bytes(B: int, L: int, H: int, D: int) -> int:
    """Device workspace bytes of the backward pass."""
    return int(_lib.load().jattn_bwd_workspace_bytes(B, L, H, D))


def fwd_workspace_bytes(B: int, L: int, H: int, D: int) -> int:
    """Device workspace bytes of the forward pass."""
    return int(_lib.load().jattn_fwd_workspace_bytes(B, L, H, D))


def backward(q, k, v, gains, out, lse, dout, valid_len=None, scale: Optional[float] = None,
             eps: float = 1e-6, dq=None, dk=None, dv=None, dgains=None, workspace=None, fwd_workspace=None):
    """Joint attention backward. Returns (dq, dk, dv bf16 [B, L, H, D], dgains fp32 [2, D]).
    fwd_workspace: the workspace returned by the forward call that produced out and lse (optional;
    the backward then reuses its normalised key rows)."""
    B, L, H, D = _check_common(q, k, v, gains, valid_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    _check_tensor("out", out, torch.bfloat16, (B, L, H, D), dev)
    _check_tensor("lse", lse, torch.float32, (B, H, L), dev)
    _check_tensor("dout", dout, torch.bfloat16, (B, L, H, D), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dgains = torch.empty(2, D, dtype=torch.float32, device=dev) if dgains is None else dgains
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (B, L, H, D), dev)
    _check_tensor("dgains", dgains, torch.float32, (2, D), dev)
    lib = _lib.load()
    need = int(lib.jattn_bwd_workspace_bytes(B, L, H, D))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.jattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(valid_len), _ptr(out), _ptr(lse),
                       _ptr(dout), B, L, H, D, ctypes.c_float(scale), ctypes.c_float(eps), _ptr(dq),
                       _ptr(dk), _ptr(dv), _ptr(dgains), _ptr(workspace), workspace.numel(), _ptr(fwd_workspace),
                       _stream(q))
    _lib.check("jattn_bwd", st)
    return dq, dk, dv, dgains


class JointAttention(torch.autograd.Function):
    """Autograd wrapper: saves the forward outputs (out, lse, the normalised keys) and calls jattn_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, gains, valid_len=None, scale=None, eps=1e-6):
        out, lse, ws = forward(q, k, v, gains, valid_len, scale, eps, return_workspace=True)
        ctx.save_for_backward(q, k, v, gains, out, lse, valid_len, ws)
        ctx.scale, ctx.eps = scale, eps
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, gains, out, lse, valid_len, ws = ctx.saved_tensors
        dq, dk, dv, dg = backward(q, k, v, gains, out, lse, dout.to(torch.bfloat16).contiguous(),
                                  valid_len, ctx.scale, ctx.eps, fwd_workspace=ws)
        return dq, dk, dv, dg, None, None, None


def joint_attention(q, k, v, gains, valid_len=None, scale=None, eps=1e-6):
    return JointAttention.apply(q, k, v, gains, valid_len, scale, eps)
