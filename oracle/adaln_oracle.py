"""fp64 CPU oracle for the adaLN-modulated QKV projection of one token stream (forward and backward).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The HIP library never calls it, shares no code with it and does not import it.

What is computed, and where the pages fix it
--------------------------------------------
[RD] = the re-diffusion README (Aaronaferns/re-diffusion). Its architecture flowchart (the DiT-layer
box) applies adaLN to each stream with the conditioning vector and then computes Q, K and V per
stream, before the joint attention; its design-notes table says the adaLN is scale + shift
(zero-initialised, no gate).

Readings where the pages are silent (each one is listed in the design document):
  * adaLN(x, t) = LN(x) * (1 + scale) + shift, with LN the LayerNorm over the C channels of a token
    without learned affine parameters (the modulation supplies them), biased variance, eps inside
    the square root. (shift, scale) is one pair of C-vectors per sample, the output of the
    conditioning linear that the pages zero-initialise; here it is an input, `mod[b] = (shift,
    scale)`.
  * QKV: one linear layer C -> 3C with bias, torch's Linear layout (weight [3C, C], y = h W^T + b);
    output columns [0, C) are q, [C, 2C) k, [2C, 3C) v, each split into H heads of D = C / H.

Backward: the analytic gradient of L = sum(q dq) + sum(k dk) + sum(v dv):
  dy = [dq | dk | dv], dW = dy^T h, db = sum over tokens of dy, dh = dy W,
  dshift_b = sum over the tokens of sample b of dh, dscale_b = the same sum of dh * xhat,
  and the LayerNorm backward with g = dh * (1 + scale):
  dx = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat)).

Every function here is pinned by tests that do not reuse it (finite differences, closed forms,
invariances, and torch's fp64 layer_norm and linear with autograd as independent routines).
"""
from __future__ import annotations

import numpy as np


def layer_norm_rows(x: np.ndarray, eps: float):
    """LayerNorm over the last axis without affine parameters: (xhat, mean, rstd)."""
    mean = x.mean(axis=-1, keepdims=True)
    xc = x - mean
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    return xc * rstd, mean[..., 0], rstd[..., 0]


def adaln_qkv_forward(x, mod, w, bias, H: int, eps: float) -> dict:
    """One stream. x [B, N, C], mod [B, 2, C] (row 0 shift, row 1 scale), w [3C, C], bias [3C] or
    None. Returns q, k, v [B, N, H, C/H], the modulated input h [B, N, C] and the LayerNorm
    statistics mean, rstd [B, N]."""
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    assert C % H == 0 and w.shape == (3 * C, C) and mod.shape == (B, 2, C)
    xhat, mean, rstd = layer_norm_rows(x, eps)
    shift, scale = mod[:, 0][:, None, :], mod[:, 1][:, None, :]
    h = xhat * (1.0 + scale) + shift
    y = h @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        y = y + bias
    D = C // H
    q, k, v = (y[..., i * C:(i + 1) * C].reshape(B, N, H, D) for i in range(3))
    return dict(q=q, k=k, v=v, h=h, xhat=xhat, mean=mean, rstd=rstd)


def adaln_qkv_backward(x, mod, w, bias, H: int, eps: float, dq, dk, dv, fwd: dict | None = None) -> dict:
    """Gradients of sum(q dq + k dk + v dv) with respect to x, mod, w and bias (dbias is returned even
    when bias is None: it is the gradient a bias would receive)."""
    f = adaln_qkv_forward(x, mod, w, bias, H, eps) if fwd is None else fwd
    B, N, C = np.shape(x)
    dy = np.concatenate([np.asarray(t, dtype=np.float64).reshape(B, N, C) for t in (dq, dk, dv)], axis=-1)
    h, xhat, rstd = f["h"], f["xhat"], f["rstd"]
    dw = dy.reshape(-1, 3 * C).T @ h.reshape(-1, C)
    dbias = dy.reshape(-1, 3 * C).sum(axis=0)
    dh = dy @ np.asarray(w, dtype=np.float64)
    dmod = np.stack([dh.sum(axis=1), (dh * xhat).sum(axis=1)], axis=1)
    g = dh * (1.0 + mod[:, 1][:, None, :])
    dx = rstd[..., None] * (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dict(dx=dx, dmod=dmod, dw=dw, dbias=dbias)


def adaln_qkv_fwd_bwd(x, mod, w, bias, H: int, eps: float, dq, dk, dv) -> dict:
    f = adaln_qkv_forward(x, mod, w, bias, H, eps)
    out = dict(f)
    out.update(adaln_qkv_backward(x, mod, w, bias, H, eps, dq, dk, dv, fwd=f))
    return out
