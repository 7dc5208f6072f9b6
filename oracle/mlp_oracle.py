"""fp64 CPU oracle for the per-stream MLP block after the joint attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The HIP library never calls it, shares no code with it and does not import it.

What is computed, and where the pages fix it
--------------------------------------------
[RD] = the re-diffusion README. Its architecture flowchart (the DiT-layer box) continues each stream
after the attention's split with fc, adaLN and a SwiGLU MLP, and one residual per stream; its
design-notes table gives the MLP as SwiGLU (SD3: GELU) and one ungated residual per block (SD3: two,
gated).

Readings where the pages are silent (each one is listed in the design document):
  * The block is  out = x + SwiGLU(adaLN(fc(o))):  o is the stream's attention output, x the stream's
    input to the layer (the one residual), fc a C -> C linear layer with bias, adaLN as in the QKV
    prologue (LayerNorm without affine parameters, then * (1 + scale) + shift with this block's own
    per-sample pair), and SwiGLU(u) = (silu(u W1^T + b1) * (u W3^T + b3)) W2^T + b2.
  * W1 and W3 are stored as one [2F, C] matrix W12 (rows [0, F) = W1, [F, 2F) = W3, bias b12 [2F])
    and W2 is [C, F]; silu(a) = a * sigmoid(a). F is the hidden width (a parameter).

Backward: the gradients of sum(out * dout) with respect to o, x, the modulation, and every weight and
bias:  dx = dout;  dW2 = dout^T hid, db2 = sum dout, dhid = dout W2;  da = dhid * g * silu'(a),
dg = dhid * silu(a), with silu'(a) = s (1 + a (1 - s)), s = sigmoid(a);  dW12 = [da|dg]^T u,
db12 = sum [da|dg], du = [da|dg] W12;  then the adaLN backward (as in the QKV prologue) gives dz and
the modulation gradient;  dWfc = dz^T o, dbfc = sum dz, do = dz Wfc.

Every function here is pinned by tests that do not reuse it (finite differences, torch's fp64
linear, layer_norm and silu with autograd, closed forms for special weights, Euler identities).
"""
from __future__ import annotations

import numpy as np

from .adaln_oracle import layer_norm_rows


def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def mlp_forward(o, x, mod, wfc, bfc, w12, b12, w2, b2, eps: float) -> dict:
    """One stream. o, x [B, N, C]; mod [B, 2, C] (shift, scale); wfc [C, C], bfc [C]; w12 [2F, C], b12 [2F];
    w2 [C, F], b2 [C]. Biases may be None. Returns out and the intermediates."""
    o = np.asarray(o, dtype=np.float64)
    B, N, C = o.shape
    F = np.shape(w12)[0] // 2
    assert np.shape(w12) == (2 * F, C) and np.shape(w2) == (C, F) and np.shape(wfc) == (C, C)
    add = lambda y, b: y if b is None else y + b
    z = add(o @ np.asarray(wfc, dtype=np.float64).T, bfc)
    zhat, mean, rstd = layer_norm_rows(z, eps)
    u = zhat * (1.0 + mod[:, 1][:, None, :]) + mod[:, 0][:, None, :]
    ag = add(u @ np.asarray(w12, dtype=np.float64).T, b12)
    a, g = ag[..., :F], ag[..., F:]
    hid = a * _sigmoid(a) * g
    y = add(hid @ np.asarray(w2, dtype=np.float64).T, b2)
    out = np.asarray(x, dtype=np.float64) + y
    return dict(out=out, y=y, z=z, zhat=zhat, mean=mean, rstd=rstd, u=u, a=a, g=g, hid=hid)


def mlp_backward(o, x, mod, wfc, bfc, w12, b12, w2, b2, eps: float, dout, fwd: dict | None = None) -> dict:
    f = mlp_forward(o, x, mod, wfc, bfc, w12, b12, w2, b2, eps) if fwd is None else fwd
    o = np.asarray(o, dtype=np.float64)
    B, N, C = o.shape
    dy = np.asarray(dout, dtype=np.float64)
    rows = lambda t: t.reshape(-1, t.shape[-1])
    dw2 = rows(dy).T @ rows(f["hid"])
    db2 = rows(dy).sum(axis=0)
    dhid = dy @ np.asarray(w2, dtype=np.float64)
    a, g = f["a"], f["g"]
    s = _sigmoid(a)
    da = dhid * g * s * (1.0 + a * (1.0 - s))
    dg = dhid * a * s
    dag = np.concatenate([da, dg], axis=-1)
    dw12 = rows(dag).T @ rows(f["u"])
    db12 = rows(dag).sum(axis=0)
    du = dag @ np.asarray(w12, dtype=np.float64)
    dmod = np.stack([du.sum(axis=1), (du * f["zhat"]).sum(axis=1)], axis=1)
    gz = du * (1.0 + mod[:, 1][:, None, :])
    zh = f["zhat"]
    dz = f["rstd"][..., None] * (gz - gz.mean(axis=-1, keepdims=True) - zh * (gz * zh).mean(axis=-1, keepdims=True))
    dwfc = rows(dz).T @ rows(o)
    dbfc = rows(dz).sum(axis=0)
    do = dz @ np.asarray(wfc, dtype=np.float64)
    return dict(do=do, dx=dy.copy(), dmod=dmod, dwfc=dwfc, dbfc=dbfc, dw12=dw12, db12=db12, dw2=dw2, db2=db2,
                dz=dz, dag=dag)


def mlp_fwd_bwd(o, x, mod, wfc, bfc, w12, b12, w2, b2, eps: float, dout) -> dict:
    f = mlp_forward(o, x, mod, wfc, bfc, w12, b12, w2, b2, eps)
    r = dict(f)
    r.update(mlp_backward(o, x, mod, wfc, bfc, w12, b12, w2, b2, eps, dout, fwd=f))
    return r
