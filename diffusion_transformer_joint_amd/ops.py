"""Python binding of libjattn.so: argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the computation runs in the
library's kernels. Layouts: q, k, v, out, dout, dq, dk, dv are bf16 [B, L, H, D] contiguous;
gains fp32 [2, D] (row 0 for Q, row 1 for K); valid_len int32 [B] (keys per sequence) or None;
lse fp32 [B, H, L] (natural-log row log-sum-exp). window (optional) = (left, right): query i sees only
keys i - left .. i + right (a negative bound is none), through jattn_fwd_window / jattn_bwd_window.

Two-stream functions (``*_streams``): each per-token tensor is an (image, text) pair of bf16 tensors
[B, N_img, H, D] and [B, N_txt, H, D] (the joint sequence is image rows then text rows, L = N_img +
N_txt); gains fp32 [2, 2, D] (gains[s, 0] = Q gain, gains[s, 1] = K gain of stream s, image = 0);
valid_len and lse as above, over the joint sequence.

Packed variable-length functions (``*_varlen``): q, k, v, out, dout, dq, dk, dv are bf16 [total, H, D]
with sequence b at rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens int32 [B + 1] on the device);
each sequence attends only to itself. lse is fp32 [total * H]: sequence b, head h, row l at
cu_seqlens[b] * H + h * L_b + l. max_seqlen (a Python int) bounds the sequence lengths.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib

__all__ = ["forward", "backward", "workspace_bytes", "fwd_workspace_bytes", "JointAttention", "joint_attention",
           "forward_streams", "backward_streams", "JointAttentionStreams", "joint_attention_streams",
           "forward_varlen", "backward_varlen", "JointAttentionVarlen", "joint_attention_varlen"]


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
            workspace: Optional[torch.Tensor] = None, return_workspace: bool = False, window=None):
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
    if window is None:
        st = lib.jattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(valid_len), B, L, H, D,
                           ctypes.c_float(scale), ctypes.c_float(eps), _ptr(out), _ptr(lse), _ptr(workspace),
                           workspace.numel(), _stream(q))
        _lib.check("jattn_fwd", st)
    else:
        st = lib.jattn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(valid_len), B, L, H, D,
                                  ctypes.c_float(scale), ctypes.c_float(eps), int(window[0]), int(window[1]), _ptr(out),
                                  _ptr(lse), _ptr(workspace), workspace.numel(), None, 0, _stream(q))
        _lib.check("jattn_fwd_window", st)
    return (out, lse, workspace) if return_workspace else (out, lse)


def workspace_bytes(B: int, L: int, H: int, D: int) -> int:
    """Device workspace bytes of the backward pass."""
    return int(_lib.load().jattn_bwd_workspace_bytes(B, L, H, D))


def fwd_workspace_bytes(B: int, L: int, H: int, D: int) -> int:
    """Device workspace bytes of the forward pass."""
    return int(_lib.load().jattn_fwd_workspace_bytes(B, L, H, D))


def backward(q, k, v, gains, out, lse, dout, valid_len=None, scale: Optional[float] = None,
             eps: float = 1e-6, dq=None, dk=None, dv=None, dgains=None, workspace=None, fwd_workspace=None,
             window=None):
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
    if window is None:
        st = lib.jattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(valid_len), _ptr(out), _ptr(lse),
                           _ptr(dout), B, L, H, D, ctypes.c_float(scale), ctypes.c_float(eps), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(dgains), _ptr(workspace), workspace.numel(), _ptr(fwd_workspace),
                           _stream(q))
        _lib.check("jattn_bwd", st)
    else:
        st = lib.jattn_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(valid_len), _ptr(out), _ptr(lse),
                                  _ptr(dout), B, L, H, D, ctypes.c_float(scale), ctypes.c_float(eps), int(window[0]),
                                  int(window[1]), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgains), _ptr(workspace),
                                  workspace.numel(), _ptr(fwd_workspace), None, 0, _stream(q))
        _lib.check("jattn_bwd_window", st)
    return dq, dk, dv, dgains


class JointAttention(torch.autograd.Function):
    """Autograd wrapper: saves the forward outputs (out, lse, the normalised keys) and calls jattn_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, gains, valid_len=None, scale=None, eps=1e-6, window=None):
        out, lse, ws = forward(q, k, v, gains, valid_len, scale, eps, return_workspace=True, window=window)
        ctx.save_for_backward(q, k, v, gains, out, lse, valid_len, ws)
        ctx.scale, ctx.eps, ctx.window = scale, eps, window
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, gains, out, lse, valid_len, ws = ctx.saved_tensors
        dq, dk, dv, dg = backward(q, k, v, gains, out, lse, dout.to(torch.bfloat16).contiguous(),
                                  valid_len, ctx.scale, ctx.eps, fwd_workspace=ws, window=ctx.window)
        return dq, dk, dv, dg, None, None, None, None


def joint_attention(q, k, v, gains, valid_len=None, scale=None, eps=1e-6, window=None):
    return JointAttention.apply(q, k, v, gains, valid_len, scale, eps, window)


# ------------------------------------------------------------------------------------------------
# Two-stream entry points

def _check_pair(name, t, dtype, B, n_img, n_txt, H, D, device):
    if not isinstance(t, (tuple, list)) or len(t) != 2:
        raise TypeError(f"{name} must be an (image, text) pair of tensors")
    _check_tensor(f"{name}[0]", t[0], dtype, (B, n_img, H, D), device)
    _check_tensor(f"{name}[1]", t[1], dtype, (B, n_txt, H, D), device)


def _pair_ptrs(t):
    return _lib.PtrPair(_ptr(t[0]) if t[0].numel() else None, _ptr(t[1]) if t[1].numel() else None)


def _check_streams(q, k, v, gains, valid_len):
    if not isinstance(q, (tuple, list)) or len(q) != 2 or q[0].dim() != 4 or q[1].dim() != 4:
        raise ValueError("q must be an (image [B, N_img, H, D], text [B, N_txt, H, D]) pair")
    B, n_img, H, D = q[0].shape
    n_txt = q[1].shape[1]
    dev = q[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_pair(name, t, torch.bfloat16, B, n_img, n_txt, H, D, dev)
    _check_tensor("gains", gains, torch.float32, (2, 2, D), dev)
    if valid_len is not None:
        _check_tensor("valid_len", valid_len, torch.int32, (B,), dev)
    return B, n_img, n_txt, H, D


def forward_streams(q, k, v, gains, valid_len=None, scale: Optional[float] = None, eps: float = 1e-6,
                    out=None, lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    return_workspace: bool = False):
    """Two-stream joint attention forward. Returns ((out_img, out_txt), lse fp32 [B, H, L]), plus the
    forward workspace if return_workspace."""
    B, n_img, n_txt, H, D = _check_streams(q, k, v, gains, valid_len)
    L = n_img + n_txt
    dev = q[0].device
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = (torch.empty_like(q[0]), torch.empty_like(q[1]))
    if lse is None:
        lse = torch.empty(B, H, L, dtype=torch.float32, device=dev)
    _check_pair("out", out, torch.bfloat16, B, n_img, n_txt, H, D, dev)
    _check_tensor("lse", lse, torch.float32, (B, H, L), dev)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(int(lib.jattn_fwd_workspace_bytes(B, L, H, D)), 1), dtype=torch.uint8, device=dev)
    qp, kp, vp, op = _pair_ptrs(q), _pair_ptrs(k), _pair_ptrs(v), _pair_ptrs(out)
    st = lib.jattn_fwd_streams(qp.arg, kp.arg, vp.arg, _ptr(gains), _ptr(valid_len), B, n_img, n_txt, H, D,
                               ctypes.c_float(scale), ctypes.c_float(eps), op.arg, _ptr(lse), _ptr(workspace),
                               workspace.numel(), None, 0, _stream(q[0]))
    _lib.check("jattn_fwd_streams", st)
    out = tuple(out)
    return (out, lse, workspace) if return_workspace else (out, lse)


def backward_streams(q, k, v, gains, out, lse, dout, valid_len=None, scale: Optional[float] = None,
                     eps: float = 1e-6, workspace=None, fwd_workspace=None):
    """Two-stream joint attention backward. Returns ((dq_img, dq_txt), (dk_img, dk_txt), (dv_img, dv_txt),
    dgains fp32 [2, 2, D])."""
    B, n_img, n_txt, H, D = _check_streams(q, k, v, gains, valid_len)
    L = n_img + n_txt
    dev = q[0].device
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check_pair("out", out, torch.bfloat16, B, n_img, n_txt, H, D, dev)
    _check_pair("dout", dout, torch.bfloat16, B, n_img, n_txt, H, D, dev)
    _check_tensor("lse", lse, torch.float32, (B, H, L), dev)
    dq = (torch.empty_like(q[0]), torch.empty_like(q[1]))
    dk = (torch.empty_like(k[0]), torch.empty_like(k[1]))
    dv = (torch.empty_like(v[0]), torch.empty_like(v[1]))
    dgains = torch.empty(2, 2, D, dtype=torch.float32, device=dev)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(int(lib.jattn_bwd_workspace_bytes(B, L, H, D)), 1), dtype=torch.uint8, device=dev)
    ptrs = [_pair_ptrs(t) for t in (q, k, v, out, dout, dq, dk, dv)]
    qp, kp, vp, op, dop, dqp, dkp, dvp = ptrs
    st = lib.jattn_bwd_streams(qp.arg, kp.arg, vp.arg, _ptr(gains), _ptr(valid_len), op.arg, _ptr(lse), dop.arg,
                               B, n_img, n_txt, H, D, ctypes.c_float(scale), ctypes.c_float(eps), dqp.arg, dkp.arg,
                               dvp.arg, _ptr(dgains), _ptr(workspace), workspace.numel(), _ptr(fwd_workspace), None,
                               0, _stream(q[0]))
    _lib.check("jattn_bwd_streams", st)
    return dq, dk, dv, dgains


class JointAttentionStreams(torch.autograd.Function):
    """Autograd wrapper of the two-stream entry points; inputs and outputs are the stream parts."""

    @staticmethod
    def forward(ctx, q_img, q_txt, k_img, k_txt, v_img, v_txt, gains, valid_len=None, scale=None, eps=1e-6):
        q, k, v = (q_img, q_txt), (k_img, k_txt), (v_img, v_txt)
        out, lse, ws = forward_streams(q, k, v, gains, valid_len, scale, eps, return_workspace=True)
        ctx.save_for_backward(q_img, q_txt, k_img, k_txt, v_img, v_txt, gains, out[0], out[1], lse, valid_len, ws)
        ctx.scale, ctx.eps = scale, eps
        return out

    @staticmethod
    def backward(ctx, d_img, d_txt):
        q_img, q_txt, k_img, k_txt, v_img, v_txt, gains, o_img, o_txt, lse, valid_len, ws = ctx.saved_tensors
        prep = lambda t, like: (torch.zeros_like(like) if t is None else t.to(torch.bfloat16).contiguous())
        dout = (prep(d_img, o_img), prep(d_txt, o_txt))
        dq, dk, dv, dg = backward_streams((q_img, q_txt), (k_img, k_txt), (v_img, v_txt), gains, (o_img, o_txt),
                                          lse, dout, valid_len, ctx.scale, ctx.eps, fwd_workspace=ws)
        return dq[0], dq[1], dk[0], dk[1], dv[0], dv[1], dg, None, None, None


def joint_attention_streams(q, k, v, gains, valid_len=None, scale=None, eps=1e-6):
    """Two-stream joint attention with autograd: q, k, v as (image, text) pairs; returns (out_img, out_txt)."""
    return JointAttentionStreams.apply(q[0], q[1], k[0], k[1], v[0], v[1], gains, valid_len, scale, eps)


# ------------------------------------------------------------------------------------------------
# Packed variable-length entry points

def _check_varlen(q, k, v, gains, cu_seqlens, max_seqlen):
    if q.dim() != 3:
        raise ValueError("q must be [total, H, D]")
    total, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, (total, H, D), dev)
    _check_tensor("gains", gains, torch.float32, (2, D), dev)
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be an int32 [B + 1] tensor")
    B = cu_seqlens.numel() - 1
    _check_tensor("cu_seqlens", cu_seqlens, torch.int32, (B + 1,), dev)
    if int(max_seqlen) < 1:
        raise ValueError("max_seqlen must be >= 1")
    return B, total, H, D


def forward_varlen(q, k, v, gains, cu_seqlens, max_seqlen: int, scale: Optional[float] = None, eps: float = 1e-6,
                   return_workspace: bool = False):
    """Packed variable-length joint attention forward. Returns (out bf16 [total, H, D], lse fp32 [total * H]),
    plus the forward workspace if return_workspace."""
    B, total, H, D = _check_varlen(q, k, v, gains, cu_seqlens, max_seqlen)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty_like(q)
    lse = torch.empty(total * H, dtype=torch.float32, device=q.device)
    lib = _lib.load()
    workspace = torch.empty(max(int(lib.jattn_varlen_fwd_workspace_bytes(B, int(max_seqlen), total, H, D)), 1),
                            dtype=torch.uint8, device=q.device)
    st = lib.jattn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(cu_seqlens), B, int(max_seqlen), total, H,
                              D, ctypes.c_float(scale), ctypes.c_float(eps), _ptr(out), _ptr(lse), _ptr(workspace),
                              workspace.numel(), None, 0, _stream(q))
    _lib.check("jattn_fwd_varlen", st)
    return (out, lse, workspace) if return_workspace else (out, lse)


def backward_varlen(q, k, v, gains, cu_seqlens, max_seqlen: int, out, lse, dout, scale: Optional[float] = None,
                    eps: float = 1e-6, fwd_workspace=None):
    """Packed variable-length joint attention backward. Returns (dq, dk, dv bf16 [total, H, D], dgains fp32 [2, D])."""
    B, total, H, D = _check_varlen(q, k, v, gains, cu_seqlens, max_seqlen)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    _check_tensor("out", out, torch.bfloat16, (total, H, D), dev)
    _check_tensor("dout", dout, torch.bfloat16, (total, H, D), dev)
    _check_tensor("lse", lse, torch.float32, (total * H,), dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dgains = torch.empty(2, D, dtype=torch.float32, device=dev)
    lib = _lib.load()
    workspace = torch.empty(max(int(lib.jattn_varlen_bwd_workspace_bytes(B, int(max_seqlen), total, H, D)), 1),
                            dtype=torch.uint8, device=dev)
    st = lib.jattn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(gains), _ptr(cu_seqlens), _ptr(out), _ptr(lse),
                              _ptr(dout), B, int(max_seqlen), total, H, D, ctypes.c_float(scale), ctypes.c_float(eps),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgains), _ptr(workspace), workspace.numel(),
                              _ptr(fwd_workspace), None, 0, _stream(q))
    _lib.check("jattn_bwd_varlen", st)
    return dq, dk, dv, dgains


class JointAttentionVarlen(torch.autograd.Function):
    """Autograd wrapper of the packed variable-length entry points."""

    @staticmethod
    def forward(ctx, q, k, v, gains, cu_seqlens, max_seqlen, scale=None, eps=1e-6):
        out, lse, ws = forward_varlen(q, k, v, gains, cu_seqlens, max_seqlen, scale, eps, return_workspace=True)
        ctx.save_for_backward(q, k, v, gains, cu_seqlens, out, lse, ws)
        ctx.max_seqlen, ctx.scale, ctx.eps = max_seqlen, scale, eps
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, gains, cu, out, lse, ws = ctx.saved_tensors
        dq, dk, dv, dg = backward_varlen(q, k, v, gains, cu, ctx.max_seqlen, out, lse,
                                         dout.to(torch.bfloat16).contiguous(), ctx.scale, ctx.eps, fwd_workspace=ws)
        return dq, dk, dv, dg, None, None, None, None


def joint_attention_varlen(q, k, v, gains, cu_seqlens, max_seqlen, scale=None, eps=1e-6):
    return JointAttentionVarlen.apply(q, k, v, gains, cu_seqlens, max_seqlen, scale, eps)
