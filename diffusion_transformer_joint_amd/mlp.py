"""Python binding of the MLP block after the attention (include/jattn_mlp.h): argument marshalling only;
every step runs in the library's kernels.

Per-stream arguments are (image, text) pairs: o, x bf16 [B, n_s, C] (attention output, the stream's input
to the layer); mod fp32 [B, 2, C] (shift, scale); wfc bf16 [C, C], bfc fp32 [C] or None; w12 bf16 [2F, C]
(rows [0, F) = W1, [F, 2F) = W3), b12 fp32 [2F] or None; w2 bf16 [C, F], b2 fp32 [C] or None.
out = x + (silu(a) * g) W2^T + b2 with [a | g] = adaLN(o Wfc^T + bfc) W12^T + b12.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from .adaln import _pair, _ptrs
from .ops import _check_tensor, _ptr, _stream

__all__ = ["mlp_forward", "mlp_backward", "MLPBlock", "mlp_block", "fwd_workspace_bytes", "bwd_workspace_bytes"]


def fwd_workspace_bytes(B: int, n_img: int, n_txt: int, C: int, F: int) -> int:
    return int(_lib.load().jattn_mlp_fwd_workspace_bytes(B, n_img, n_txt, C, F))


def bwd_workspace_bytes(B: int, n_img: int, n_txt: int, C: int, F: int) -> int:
    return int(_lib.load().jattn_mlp_bwd_workspace_bytes(B, n_img, n_txt, C, F))


def _sizes(o, w12):
    o = _pair(o)
    if o[0].dim() != 3 or o[1].dim() != 3:
        raise ValueError("o must be an (image [B, n_img, C], text [B, n_txt, C]) pair")
    B, n_img, C = o[0].shape
    F = _pair(w12)[0].shape[0] // 2
    return B, n_img, o[1].shape[1], C, F, o[0].device


def _bias_pair(b):
    return (None, None) if b is None else _pair(b)


def mlp_forward(o, x, mod, wfc, w12, w2, bfc=None, b12=None, b2=None, eps: float = 1e-6,
                workspace: Optional[torch.Tensor] = None, events=None):
    """Returns ((out_img, out_txt), workspace); keep the workspace for the backward pass."""
    B, n_img, n_txt, C, F, dev = _sizes(o, w12)
    ns = (n_img, n_txt)
    o, x, mod, wfc, w12, w2 = (_pair(t) for t in (o, x, mod, wfc, w12, w2))
    bfc, b12, b2 = (_bias_pair(t) for t in (bfc, b12, b2))
    for s in range(2):
        _check_tensor(f"o[{s}]", o[s], torch.bfloat16, (B, ns[s], C), dev)
        _check_tensor(f"x[{s}]", x[s], torch.bfloat16, (B, ns[s], C), dev)
        _check_tensor(f"mod[{s}]", mod[s], torch.float32, (B, 2, C), dev)
        _check_tensor(f"wfc[{s}]", wfc[s], torch.bfloat16, (C, C), dev)
        _check_tensor(f"w12[{s}]", w12[s], torch.bfloat16, (2 * F, C), dev)
        _check_tensor(f"w2[{s}]", w2[s], torch.bfloat16, (C, F), dev)
        for name, b, n in (("bfc", bfc, C), ("b12", b12, 2 * F), ("b2", b2, C)):
            if b[s] is not None:
                _check_tensor(f"{name}[{s}]", b[s], torch.float32, (n,), dev)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(fwd_workspace_bytes(B, n_img, n_txt, C, F), 1), dtype=torch.uint8, device=dev)
    out = tuple(torch.empty(B, n, C, dtype=torch.bfloat16, device=dev) for n in ns)
    bp = [_lib.PtrPair(*(None if t is None else t.data_ptr() for t in b)) for b in (bfc, b12, b2)]
    op, xp, mp, wfp, w12p, w2p, outp = (_ptrs(t) for t in (o, x, mod, wfc, w12, w2, out))
    ev, nev = _lib.event_array(events)
    st = lib.jattn_mlp_fwd(op.arg, xp.arg, mp.arg, wfp.arg, bp[0].arg, w12p.arg, bp[1].arg, w2p.arg, bp[2].arg, B,
                           n_img, n_txt, C, F, ctypes.c_float(eps), outp.arg, _ptr(workspace), workspace.numel(), ev,
                           nev, _stream(o[0]))
    _lib.check("jattn_mlp_fwd", st)
    return out, workspace


def mlp_backward(o, mod, wfc, w12, w2, dout, fwd_workspace: torch.Tensor, need_dbias: bool = True,
                 workspace: Optional[torch.Tensor] = None, events=None):
    """Returns dict of (image, text) pairs: do, dmod, dwfc, dw12, dw2 and (if need_dbias) dbfc, db12, db2.
    The gradient of x is dout itself."""
    B, n_img, n_txt, C, F, dev = _sizes(o, w12)
    ns = (n_img, n_txt)
    o, mod, wfc, w12, w2, dout = (_pair(t) for t in (o, mod, wfc, w12, w2, dout))
    for s in range(2):
        _check_tensor(f"dout[{s}]", dout[s], torch.bfloat16, (B, ns[s], C), dev)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, n_img, n_txt, C, F), 1), dtype=torch.uint8, device=dev)
    f32 = lambda *shape: tuple(torch.empty(*shape, dtype=torch.float32, device=dev) for _ in ns)
    g = dict(do=tuple(torch.empty(B, n, C, dtype=torch.bfloat16, device=dev) for n in ns), dmod=f32(B, 2, C),
             dwfc=f32(C, C), dw12=f32(2 * F, C), dw2=f32(C, F))
    if need_dbias:
        g.update(dbfc=f32(C), db12=f32(2 * F), db2=f32(C))
    none = _lib.PtrPair(None, None)
    pp = {k: _ptrs(v) for k, v in g.items()}
    ins = [_ptrs(t) for t in (o, mod, wfc, w12, w2, dout)]
    ev, nev = _lib.event_array(events)
    st = lib.jattn_mlp_bwd(*(p.arg for p in ins), B, n_img, n_txt, C, F, pp["do"].arg, pp["dmod"].arg, pp["dwfc"].arg,
                           pp.get("dbfc", none).arg, pp["dw12"].arg, pp.get("db12", none).arg, pp["dw2"].arg,
                           pp.get("db2", none).arg, _ptr(fwd_workspace), fwd_workspace.numel(), _ptr(workspace),
                           workspace.numel(), ev, nev, _stream(o[0]))
    _lib.check("jattn_mlp_bwd", st)
    return g


class MLPBlock(torch.autograd.Function):
    """Autograd wrapper over the stream parts; weight gradients come back fp32 and are cast to the
    weights' dtype."""

    @staticmethod
    def forward(ctx, o0, o1, x0, x1, m0, m1, wfc0, wfc1, bfc0, bfc1, w120, w121, b120, b121, w20, w21, b20, b21,
                eps=1e-6):
        bias = lambda a, b: None if a is None and b is None else (a, b)
        out, ws = mlp_forward((o0, o1), (x0, x1), (m0, m1), (wfc0, wfc1), (w120, w121), (w20, w21), bias(bfc0, bfc1),
                              bias(b120, b121), bias(b20, b21), eps)
        ctx.save_for_backward(o0, o1, m0, m1, wfc0, wfc1, w120, w121, w20, w21, ws)
        ctx.has_bias = [t is not None for t in (bfc0, bfc1, b120, b121, b20, b21)]
        return out

    @staticmethod
    def backward(ctx, d0, d1):
        o0, o1, m0, m1, wfc0, wfc1, w120, w121, w20, w21, ws = ctx.saved_tensors
        fix = lambda d, like: (torch.zeros_like(like) if d is None else d.to(torch.bfloat16).contiguous())
        dout = (fix(d0, o0), fix(d1, o1))
        g = mlp_backward((o0, o1), (m0, m1), (wfc0, wfc1), (w120, w121), (w20, w21), dout, ws,
                         need_dbias=any(ctx.has_bias))
        hb = ctx.has_bias
        db = lambda key, s, k: (g[key][s] if key in g and hb[k] else None)
        cast = lambda t, like: t.to(like.dtype)
        return (g["do"][0], g["do"][1], dout[0], dout[1], g["dmod"][0], g["dmod"][1], cast(g["dwfc"][0], wfc0),
                cast(g["dwfc"][1], wfc1), db("dbfc", 0, 0), db("dbfc", 1, 1), cast(g["dw12"][0], w120),
                cast(g["dw12"][1], w121), db("db12", 0, 2), db("db12", 1, 3), cast(g["dw2"][0], w20),
                cast(g["dw2"][1], w21), db("db2", 0, 4), db("db2", 1, 5), None)


def mlp_block(o, x, mod, wfc, w12, w2, bfc=None, b12=None, b2=None, eps: float = 1e-6):
    """The MLP block of both streams with autograd; returns (out_img, out_txt)."""
    b = lambda t: (None, None) if t is None else _pair(t)
    bf, b1, b2_ = b(bfc), b(b12), b(b2)
    return MLPBlock.apply(o[0], o[1], x[0], x[1], mod[0], mod[1], wfc[0], wfc[1], bf[0], bf[1], w12[0], w12[1], b1[0],
                          b1[1], w2[0], w2[1], b2_[0], b2_[1], eps)
