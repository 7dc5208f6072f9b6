"""fp64 CPU oracle for QK-RMSNorm joint image+text attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The HIP library never calls it, shares no code with it and does not import it.

What is computed, and where the pages fix it
--------------------------------------------
[RD] = the re-diffusion README (Aaronaferns/re-diffusion): a 254.5M MM-DiT trained with rectified
flow. [DP] = the diffusion-pipe repository summary (tdrussell/diffusion-pipe).

* Joint attention: image tokens and text tokens of one sample are concatenated into one sequence
  and a single non-causal multi-head softmax attention runs over it ([RD] headline feature list;
  architecture flowchart, the DiT-layer box: per-stream QKV, concat, joint MHSA, split).
* QK-RMSNorm: Q and K are RMS-normalised with learned gains before the product ([RD] feature list;
  design-notes table, "QK norm" row). Normalisation is over the head dim D of each (token, head)
  row; the gain is a length-D vector; Q and K have separate gains (row 0 and row 1 of ``gains``).
* The "manual attention" of [RD]'s profiling section builds the full score matrix, applies the
  softmax in fp32 and multiplies by V. That plain definition is what this oracle computes, in fp64,
  one (batch, head) pair at a time: S = scale * Qn Kn^T, P = softmax(S), O = P V.
* Key padding: keys at positions >= valid_len[b] are excluded from the softmax ([DP], the attention
  wrapper's varlen path). Padded query rows are still computed over the valid keys.
* Local window (optional): query i sees only keys i - left <= j <= i + right ([DP], the wrapper's
  windowed attention; the bounds are read as those of a sliding window, a negative bound meaning
  none). A row with no key left gets O = 0, LSE = -inf and zero gradients, as with valid_len 0.

Readings where the pages are silent (each one is listed in the design document):
  eps sits inside the square root, rms = sqrt(mean(x^2) + eps); the softmax scale multiplies the
  normalised scores; LSE is the natural-log row log-sum-exp of the scaled scores over valid keys;
  a row with no valid key gives O = 0, LSE = -inf and zero gradients; valid_len is clamped to [0, L].

Backward: the analytic gradient of L = sum(O * dO) with respect to q, k, v and both gain rows:
  dV = P^T dO, dP = dO V^T, Delta_i = sum_j P_ij dP_ij, dS = P * (dP - Delta),
  dQn = scale dS Kn, dKn = scale dS^T Qn, and the RMSNorm backward
  dx = r (g * dxn) - x (r^3 / D) sum_d(g * dxn * x),   dg = sum over rows of dxn * x * r.

Every function here is pinned by tests that do not reuse it (finite differences, closed forms,
invariances, and torch's fp64 scaled_dot_product_attention with autograd as an independent routine).
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = ["rmsnorm", "head_forward", "head_backward", "attention_forward", "attention_backward",
           "attention_fwd_bwd", "streams_fwd_bwd", "varlen_fwd_bwd"]


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """RMS-normalise each row of x [N, D] over D and multiply by the gain g [D].
    Returns (xn [N, D], r [N, 1]) with r = 1 / sqrt(mean_d x^2 + eps)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g, r


def _valid_keys(valid_len, b: int, L: int) -> int:
    if valid_len is None:
        return L
    return int(min(max(int(valid_len[b]), 0), L))


def head_forward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, gq: np.ndarray, gk: np.ndarray,
                 n: int, scale: float, eps: float, window: Optional[Tuple[int, int]] = None) -> dict:
    """One (batch, head) pair. Q, K, V: [L, D] fp64; n valid keys.
    Returns the explicit intermediates: Qn, Kn, rq, rk, S (masked with -inf), P, O, lse.
    window = (left, right): query i also sees only keys i - left <= j <= i + right (a negative bound
    is no bound); a row left with no key gets P = 0, O = 0 and lse = -inf."""
    L = Q.shape[0]
    Qn, rq = rmsnorm(Q, gq, eps)
    Kn, rk = rmsnorm(K, gk, eps)
    S = scale * (Qn @ Kn.T)
    S[:, n:] = -np.inf
    if window is not None:
        return _windowed_softmax(Qn, Kn, rq, rk, S, V, n, window)
    if n == 0:
        P = np.zeros((L, L))
        O = np.zeros_like(V)
        lse = np.full(L, -np.inf)
    else:
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        den = E.sum(axis=1, keepdims=True)
        P = E / den
        O = P @ V
        lse = (m + np.log(den))[:, 0]
    return dict(Qn=Qn, Kn=Kn, rq=rq, rk=rk, S=S, P=P, O=O, lse=lse)


def _windowed_softmax(Qn, Kn, rq, rk, S, V, n, window) -> dict:
    """The softmax and PV product of head_forward under a local window: every row over its own set of
    allowed keys, rows without one left at zero."""
    L = S.shape[0]
    left, right = window
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    allowed = j < n
    if left >= 0:
        allowed = allowed & (j >= i - left)
    if right >= 0:
        allowed = allowed & (j <= i + right)
    S = np.where(allowed, S, -np.inf)
    has = allowed.any(axis=1)
    m = np.where(has, np.max(S, axis=1), 0.0)[:, None]
    E = np.where(allowed, np.exp(S - m), 0.0)
    den = E.sum(axis=1, keepdims=True)
    P = np.where(has[:, None], E / np.where(den > 0, den, 1.0), 0.0)
    O = P @ V
    lse = np.where(has, m[:, 0] + np.log(np.where(has, den[:, 0], 1.0)), -np.inf)
    return dict(Qn=Qn, Kn=Kn, rq=rq, rk=rk, S=S, P=P, O=O, lse=lse)


def _rmsnorm_backward(x: np.ndarray, r: np.ndarray, g: np.ndarray, dxn: np.ndarray):
    """Gradient through xn = x * r * g for one set of rows: returns (dx, dg)."""
    D = x.shape[-1]
    gd = g * dxn
    dx = r * gd - x * (r ** 3 / D) * np.sum(gd * x, axis=-1, keepdims=True)
    dg = np.sum(dxn * x * r, axis=0)
    return dx, dg


def head_backward(Q, K, V, gq, gk, dO, n: int, scale: float, eps: float, fwd: Optional[dict] = None,
                  window: Optional[Tuple[int, int]] = None):
    """Analytic backward for one (batch, head) pair. Returns (dQ, dK, dV, dgq, dgk, extras)."""
    f = head_forward(Q, K, V, gq, gk, n, scale, eps, window) if fwd is None else fwd
    P = f["P"]
    dV = P.T @ dO
    dP = dO @ V.T
    delta = np.sum(P * dP, axis=1, keepdims=True)
    dS = P * (dP - delta)
    dQn = scale * (dS @ f["Kn"])
    dKn = scale * (dS.T @ f["Qn"])
    dQ, dgq = _rmsnorm_backward(Q, f["rq"], gq, dQn)
    dK, dgk = _rmsnorm_backward(K, f["rk"], gk, dKn)
    return dQ, dK, dV, dgq, dgk, dict(dS=dS, dP=dP, delta=delta[:, 0], dQn=dQn, dKn=dKn)


def _pairs(B: int, H: int, pairs: Optional[Iterable[Tuple[int, int]]]):
    return [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)


def attention_forward(q, k, v, gains, valid_len=None, scale: float = None, eps: float = 1e-6,
                      pairs: Optional[Sequence[Tuple[int, int]]] = None, window: Optional[Tuple[int, int]] = None):
    """q, k, v: [B, L, H, D] (any float dtype, promoted to fp64); gains [2, D].
    Returns out [B, L, H, D] and lse [B, H, L] (natural log) in fp64. With ``pairs`` only those
    (b, h) pairs are computed and the rest of the outputs is NaN. ``window`` as in head_forward."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    gains = np.asarray(gains, dtype=np.float64)
    B, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, L, H, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b, h in _pairs(B, H, pairs):
        f = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], gains[0], gains[1],
                         _valid_keys(valid_len, b, L), scale, eps, window)
        out[b, :, h] = f["O"]
        lse[b, h] = f["lse"]
    return out, lse


def attention_backward(q, k, v, gains, dout, valid_len=None, scale: float = None, eps: float = 1e-6,
                       pairs: Optional[Sequence[Tuple[int, int]]] = None, window: Optional[Tuple[int, int]] = None):
    """Gradients of sum(out * dout). Returns dq, dk, dv [B, L, H, D] and dgains [2, D] (fp64).
    With ``pairs`` the per-token gradients outside those pairs are NaN and dgains sums over the
    chosen pairs only."""
    return _fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps, pairs, window)[2:]


def attention_fwd_bwd(q, k, v, gains, dout, valid_len=None, scale: float = None, eps: float = 1e-6,
                      pairs: Optional[Sequence[Tuple[int, int]]] = None,
                      window: Optional[Tuple[int, int]] = None) -> dict:
    """Forward and backward in one pass over the (b, h) pairs. ``window`` as in head_forward."""
    out, lse, dq, dk, dv, dg = _fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps, pairs, window)
    return dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv, dgains=dg)


def _fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps, pairs, window=None):
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    gains = np.asarray(gains, dtype=np.float64)
    B, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, L, H, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    dq, dk, dv = (np.full((B, L, H, D), np.nan) for _ in range(3))
    dg = np.zeros((2, D))
    for b, h in _pairs(B, H, pairs):
        n = _valid_keys(valid_len, b, L)
        Q, K, V, dO = q[b, :, h], k[b, :, h], v[b, :, h], dout[b, :, h]
        f = head_forward(Q, K, V, gains[0], gains[1], n, scale, eps, window)
        dQ, dK, dV, dgq, dgk, _ = head_backward(Q, K, V, gains[0], gains[1], dO, n, scale, eps, fwd=f)
        out[b, :, h], lse[b, h] = f["O"], f["lse"]
        dq[b, :, h], dk[b, :, h], dv[b, :, h] = dQ, dK, dV
        dg[0] += dgq
        dg[1] += dgk
    return out, lse, dq, dk, dv, dg


# ------------------------------------------------------------------------------------------------
# Two-stream form. [RD]'s DiT-layer box projects Q, K and V separately for the image stream x and
# the text stream c ("QKV each"), concatenates the two streams, runs the joint attention and splits
# the result back per stream. Here each stream keeps its own tensors and its own QK-norm gains (a
# norm attached to each stream's projection; [RD]'s design-notes table names RMSNorm on Q and K
# without saying whether the streams share it). Rows are concatenated image first, so valid_len is
# still a prefix length of the joint sequence.

def _stream_of_rows(n_img: int, L: int) -> np.ndarray:
    """Stream index (0 = image, 1 = text) of each joint row."""
    return (np.arange(L) >= n_img).astype(np.int64)


def streams_fwd_bwd(q, k, v, gains, dout, valid_len=None, scale: float = None, eps: float = 1e-6,
                    pairs: Optional[Sequence[Tuple[int, int]]] = None) -> dict:
    """q, k, v, dout: (image [B, N_img, H, D], text [B, N_txt, H, D]) pairs; gains [2, 2, D] with
    gains[s, 0] the Q gain and gains[s, 1] the K gain of stream s. Concatenates each pair along the
    token axis (image first), runs the joint attention with every row normalised by its own stream's
    gains, and splits the per-token results back.
    Returns dict(out, dq, dk, dv) as (image, text) pairs, lse [B, H, N_img + N_txt] (joint row order)
    and dgains [2, 2, D] (fp64). ``pairs`` as in attention_forward."""
    cat = lambda t: np.concatenate([np.asarray(t[0], dtype=np.float64), np.asarray(t[1], dtype=np.float64)],
                                   axis=1)
    qj, kj, vj, doj = cat(q), cat(k), cat(v), cat(dout)
    gains = np.asarray(gains, dtype=np.float64)
    B, L, H, D = qj.shape
    n_img = np.asarray(q[0]).shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    stream = _stream_of_rows(n_img, L)
    gq_rows, gk_rows = gains[stream, 0], gains[stream, 1]  # [L, D] each
    out = np.full((B, L, H, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    dq, dk, dv = (np.full((B, L, H, D), np.nan) for _ in range(3))
    dg = np.zeros((2, 2, D))
    for b, h in _pairs(B, H, pairs):
        n = _valid_keys(valid_len, b, L)
        Q, K, V, dO = qj[b, :, h], kj[b, :, h], vj[b, :, h], doj[b, :, h]
        f = head_forward(Q, K, V, gq_rows, gk_rows, n, scale, eps)
        dQ, dK, dV, _, _, ex = head_backward(Q, K, V, gq_rows, gk_rows, dO, n, scale, eps, fwd=f)
        out[b, :, h], lse[b, h] = f["O"], f["lse"]
        dq[b, :, h], dk[b, :, h], dv[b, :, h] = dQ, dK, dV
        # gain gradients: each row's term dxn * x * r goes to its own stream's gain
        tq = ex["dQn"] * Q * f["rq"]
        tk = ex["dKn"] * K * f["rk"]
        for s in (0, 1):
            rows = stream == s
            dg[s, 0] += tq[rows].sum(axis=0)
            dg[s, 1] += tk[rows].sum(axis=0)
    split = lambda t: (t[:, :n_img], t[:, n_img:])
    return dict(out=split(out), lse=lse, dq=split(dq), dk=split(dk), dv=split(dv), dgains=dg)


# ------------------------------------------------------------------------------------------------
# Packed variable-length form. [DP]'s attention wrapper has a variable-length path beside the padded
# one: sequences of different lengths stored back to back, each attending only to itself. Sequence b
# holds rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the [total, H, D] tensors; all of its keys are
# valid.

def varlen_fwd_bwd(q, k, v, gains, dout, cu_seqlens, scale: float = None, eps: float = 1e-6,
                   seqs: Optional[Sequence[int]] = None) -> dict:
    """q, k, v, dout: [total, H, D]; gains [2, D]; cu_seqlens: B + 1 non-decreasing offsets starting at
    0. Runs the joint attention on every sequence separately. Returns out, dq, dk, dv [total, H, D]
    (NaN on rows of sequences not computed), lse as a list of [H, L_b] arrays (None for sequences not
    computed) and dgains [2, D] summed over the computed sequences. ``seqs`` limits the work to those
    sequences."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    gains = np.asarray(gains, dtype=np.float64)
    cu = [int(c) for c in cu_seqlens]
    B = len(cu) - 1
    total, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out, dq, dk, dv = (np.full((total, H, D), np.nan) for _ in range(4))
    lse = [None] * B
    dg = np.zeros((2, D))
    for b in (range(B) if seqs is None else seqs):
        r0, r1 = cu[b], cu[b + 1]
        n = r1 - r0
        lse[b] = np.zeros((H, n))
        for h in range(H):
            Q, K, V, dO = q[r0:r1, h], k[r0:r1, h], v[r0:r1, h], dout[r0:r1, h]
            f = head_forward(Q, K, V, gains[0], gains[1], n, scale, eps)
            dQ, dK, dV, dgq, dgk, _ = head_backward(Q, K, V, gains[0], gains[1], dO, n, scale, eps, fwd=f)
            out[r0:r1, h], lse[b][h] = f["O"], f["lse"]
            dq[r0:r1, h], dk[r0:r1, h], dv[r0:r1, h] = dQ, dK, dV
            dg[0] += dgq
            dg[1] += dgk
    return dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv, dgains=dg)
