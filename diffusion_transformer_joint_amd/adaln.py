"""Python binding of the adaLN-modulated QKV projection (include/jattn_adaln.h): argument marshalling
only; every step runs in the library's kernels.

Per-stream arguments are (image, text) pairs: x bf16 [B, n_s, C]; mod fp32 [B, 2, C] (row 0 shift,
row 1 scale); w bf16 [3C, C] (torch Linear layout); bias fp32 [3C] or None. The outputs q, k, v are
bf16 [B, n_s, H, C/H] pairs, the layout the two-stream attention entry points read. A stream with
n_s = 0 is allowed (its tensors are empty).
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from .ops import _check_tensor, _ptr, _stream

__all__ = ["adaln_qkv_forward", "adaln_qkv_backward", "AdaLNQKV", "adaln_qkv", "fwd_workspace_bytes",
           "bwd_workspace_bytes"]


def _pair(t):
    if not isinstance(t, (tuple, list)) or len(t) != 2:
        raise TypeError("expected an (image, text) pair")
    return tuple(t)


def _ptrs(t):
    return _lib.PtrPair(*(None if (u is None or u.numel() == 0) else u.data_ptr() for u in t))


def _sizes(x):
    x = _pair(x)
    if x[0].dim() != 3 or x[1].dim() != 3:
        raise ValueError("x must be an (image [B, n_img, C], text [B, n_txt, C]) pair")
    B, n_img, C = x[0].shape
    return B, n_img, x[1].shape[1], C, x[0].device


def fwd_workspace_bytes(B: int, n_img: int, n_txt: int, C: int) -> int:
    return int(_lib.load().jattn_adaln_qkv_fwd_workspace_bytes(B, n_img, n_txt, C))


def bwd_workspace_bytes(B: int, n_img: int, n_txt: int, C: int) -> int:
    return int(_lib.load().jattn_adaln_qkv_bwd_workspace_bytes(B, n_img, n_txt, C))


def adaln_qkv_forward(x, mod, w, bias=None, eps: float = 1e-6, heads: int = 1,
                      workspace: Optional[torch.Tensor] = None, events=None):
    """Returns ((q_img, q_txt), (k_img, k_txt), (v_img, v_txt), workspace); keep the workspace for the
    backward pass. `events`: optional list of torch.cuda.Event recorded after each kernel."""
    B, n_img, n_txt, C, dev = _sizes(x)
    ns = (n_img, n_txt)
    mod, w = _pair(mod), _pair(w)
    bias = (None, None) if bias is None else _pair(bias)
    if C % heads:
        raise ValueError("heads must divide C")
    for s in range(2):
        _check_tensor(f"x[{s}]", x[s], torch.bfloat16, (B, ns[s], C), dev)
        _check_tensor(f"mod[{s}]", mod[s], torch.float32, (B, 2, C), dev)
        _check_tensor(f"w[{s}]", w[s], torch.bfloat16, (3 * C, C), dev)
        if bias[s] is not None:
            _check_tensor(f"bias[{s}]", bias[s], torch.float32, (3 * C,), dev)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(fwd_workspace_bytes(B, n_img, n_txt, C), 1), dtype=torch.uint8, device=dev)
    D = C // heads
    q, k, v = ([torch.empty(B, n, heads, D, dtype=torch.bfloat16, device=dev) for n in ns] for _ in range(3))
    bp = _lib.PtrPair(*(None if b is None else b.data_ptr() for b in bias))
    xp, mp, wp, qp, kp, vp = _ptrs(x), _ptrs(mod), _ptrs(w), _ptrs(q), _ptrs(k), _ptrs(v)
    ev, nev = _lib.event_array(events)
    st = lib.jattn_adaln_qkv_fwd(xp.arg, mp.arg, wp.arg, bp.arg, B, n_img, n_txt, C, ctypes.c_float(eps), qp.arg,
                                 kp.arg, vp.arg, _ptr(workspace), workspace.numel(), ev, nev, _stream(x[0]))
    _lib.check("jattn_adaln_qkv_fwd", st)
    return tuple(q), tuple(k), tuple(v), workspace


def adaln_qkv_backward(x, mod, w, dq, dk, dv, fwd_workspace: torch.Tensor, need_dbias: bool = True,
                       workspace: Optional[torch.Tensor] = None, events=None):
    """Returns ((dx_img, dx_txt), (dmod_img, dmod_txt), (dw_img, dw_txt), (dbias_img, dbias_txt) or None).
    dq, dk, dv: (image, text) pairs of bf16 [B, n_s, C] or [B, n_s, H, D]."""
    B, n_img, n_txt, C, dev = _sizes(x)
    ns = (n_img, n_txt)
    mod, w = _pair(mod), _pair(w)
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        t = _pair(t)
        for s in range(2):
            if t[s].numel() != B * ns[s] * C or t[s].dtype != torch.bfloat16 or not t[s].is_contiguous():
                raise ValueError(f"{name}[{s}] must be a contiguous bf16 tensor of B * n_s * C elements")
        grads.append(t)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, n_img, n_txt, C), 1), dtype=torch.uint8, device=dev)
    dx = tuple(torch.empty(B, n, C, dtype=torch.bfloat16, device=dev) for n in ns)
    dmod = tuple(torch.empty(B, 2, C, dtype=torch.float32, device=dev) for _ in ns)
    dw = tuple(torch.empty(3 * C, C, dtype=torch.float32, device=dev) for _ in ns)
    dbias = tuple(torch.empty(3 * C, dtype=torch.float32, device=dev) for _ in ns) if need_dbias else None
    ptrs = [_ptrs(t) for t in (x, mod, w, *grads, dx, dmod, dw)]
    dbp = _ptrs(dbias) if need_dbias else _lib.PtrPair(None, None)
    ev, nev = _lib.event_array(events)
    st = lib.jattn_adaln_qkv_bwd(*(p.arg for p in ptrs[:6]), B, n_img, n_txt, C, *(p.arg for p in ptrs[6:]), dbp.arg,
                                 _ptr(fwd_workspace), fwd_workspace.numel(), _ptr(workspace), workspace.numel(), ev,
                                 nev, _stream(x[0]))
    _lib.check("jattn_adaln_qkv_bwd", st)
    return dx, dmod, dw, dbias


class AdaLNQKV(torch.autograd.Function):
    """Autograd wrapper: inputs and outputs are the stream parts. The weight gradients come back fp32
    and are cast to the weights' dtype."""

    @staticmethod
    def forward(ctx, x_img, x_txt, mod_img, mod_txt, w_img, w_txt, b_img, b_txt, eps=1e-6, heads=1):
        q, k, v, ws = adaln_qkv_forward((x_img, x_txt), (mod_img, mod_txt), (w_img, w_txt),
                                        None if b_img is None and b_txt is None else (b_img, b_txt), eps, heads)
        ctx.save_for_backward(x_img, x_txt, mod_img, mod_txt, w_img, w_txt, ws)
        ctx.has_bias = (b_img is not None, b_txt is not None)
        return q[0], q[1], k[0], k[1], v[0], v[1]

    @staticmethod
    def backward(ctx, dq0, dq1, dk0, dk1, dv0, dv1):
        x0, x1, m0, m1, w0, w1, ws = ctx.saved_tensors
        fix = lambda g, like: (torch.zeros(like.shape[0], like.shape[1], like.shape[2], dtype=torch.bfloat16,
                                           device=like.device) if g is None else g.to(torch.bfloat16).contiguous())
        dq = (fix(dq0, x0), fix(dq1, x1))
        dk = (fix(dk0, x0), fix(dk1, x1))
        dv = (fix(dv0, x0), fix(dv1, x1))
        dx, dmod, dw, db = adaln_qkv_backward((x0, x1), (m0, m1), (w0, w1), dq, dk, dv, ws,
                                              need_dbias=any(ctx.has_bias))
        dbs = (db[0] if ctx.has_bias[0] else None, db[1] if ctx.has_bias[1] else None) if db else (None, None)
        return dx[0], dx[1], dmod[0], dmod[1], dw[0].to(w0.dtype), dw[1].to(w1.dtype), dbs[0], dbs[1], None, None


def adaln_qkv(x, mod, w, bias=None, eps: float = 1e-6, heads: int = 1):
    """adaLN-modulated QKV projection of both streams with autograd; returns (q, k, v) pairs."""
    b = (None, None) if bias is None else _pair(bias)
    o = AdaLNQKV.apply(x[0], x[1], mod[0], mod[1], w[0], w[1], b[0], b[1], eps, heads)
    return (o[0], o[1]), (o[2], o[3]), (o[4], o[5])
