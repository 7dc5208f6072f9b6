"""Pins for the fp64 oracle. None of these re-types the oracle's formulas: each checks it against
something fixed independently of it -- finite differences, closed forms worked by hand, invariances
that the definition implies, and torch's fp64 scaled_dot_product_attention + autograd.

Sources for the definition: re-diffusion README (joint attention over concatenated image and text
tokens; QK-RMSNorm row of the design-notes table; the manual-attention description in the
profiling section) and the diffusion-pipe summary (varlen / key-padding path of its attention
wrapper)."""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import attention_backward, attention_forward, attention_fwd_bwd, head_forward

def rand_case(B=2, L=6, H=2, D=4, seed=0, gain_std=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, H, D))
    k = rng.standard_normal((B, L, H, D))
    v = rng.standard_normal((B, L, H, D))
    gains = 1.0 + gain_std * rng.standard_normal((2, D))
    dout = rng.standard_normal((B, L, H, D))
    return q, k, v, gains, dout


def loss(q, k, v, gains, dout, valid_len, scale, eps):
    out, _ = attention_forward(q, k, v, gains, valid_len, scale, eps)
    return float(np.sum(out * dout))


# ---------------------------------------------------------------- finite differences (backward)
@pytest.mark.parametrize("valid_len", [None, [5, 2]])
def test_finite_difference_gradients(valid_len):
    B, L, H, D = 2, 5, 2, 4
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=1)
    scale, eps = 0.7, 1e-3
    dq, dk, dv, dg = attention_backward(q, k, v, gains, dout, valid_len, scale, eps)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("gains", gains, dg)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v, gains, dout, valid_len, scale, eps)
            x[idx] = old - h
            lm = loss(q, k, v, gains, dout, valid_len, scale, eps)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


# ---------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("valid_len", [None, [7, 3]])
def test_matches_torch_sdpa_fp64(valid_len):
    B, L, H, D = 2, 7, 3, 8
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=2)
    scale, eps = 0.4, 1e-6
    got = attention_fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps)

    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tg = torch.tensor(gains, dtype=torch.float64, requires_grad=True)
    nq = torch.nn.functional.rms_norm(tq, (D,), weight=tg[0], eps=eps)
    nk = torch.nn.functional.rms_norm(tk, (D,), weight=tg[1], eps=eps)
    # [B, L, H, D] -> [B, H, L, D]
    Q, K, V = (t.permute(0, 2, 1, 3) for t in (nq, nk, tv))
    mask = None
    if valid_len is not None:
        mask = torch.zeros(B, 1, L, L, dtype=torch.bool)
        for b, n in enumerate(valid_len):
            mask[b, :, :, :n] = True
    O = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    O = O.permute(0, 2, 1, 3)
    O.backward(torch.tensor(dout))
    np.testing.assert_allclose(got["out"], O.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dq"], tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["dk"], tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["dv"], tv.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["dgains"], tg.grad.numpy(), rtol=1e-9, atol=1e-11)
    # LSE against scipy's logsumexp of the explicit (masked) score matrix built by torch
    S = torch.matmul(Q, K.transpose(-1, -2).contiguous()).detach().numpy() * scale
    if valid_len is not None:
        for b, n in enumerate(valid_len):
            S[b, :, :, n:] = -np.inf
    np.testing.assert_allclose(got["lse"], scipy.special.logsumexp(S, axis=-1), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_closed_form_one_dim_two_tokens():
    """D = 1, eps = 0: RMSNorm of a scalar is sign(x) * g, so with q = (1, -2), k = (3, -0.5),
    gains (2, 1.5) and scale 0.5 the normalised scores are S = 1.5 * [[1, -1], [-1, 1]]. Each row is a
    two-term softmax: P = (sigmoid(3), sigmoid(-3)) for row 0 and reversed for row 1, and both rows
    have LSE = 1.5 + log(1 + exp(-3)). Worked by hand, not by the oracle's formulas."""
    q = np.array([1.0, -2.0]).reshape(1, 2, 1, 1)
    k = np.array([3.0, -0.5]).reshape(1, 2, 1, 1)
    v = np.array([0.7, -1.1]).reshape(1, 2, 1, 1)
    gains = np.array([[2.0], [1.5]])
    out, lse = attention_forward(q, k, v, gains, None, 0.5, 0.0)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    expected_out = [sig(3) * 0.7 + sig(-3) * -1.1, sig(-3) * 0.7 + sig(3) * -1.1]
    expected_lse = 1.5 + math.log1p(math.exp(-3.0))
    np.testing.assert_allclose(out.reshape(2), expected_out, rtol=1e-14)
    np.testing.assert_allclose(lse.reshape(2), [expected_lse, expected_lse], rtol=1e-14)


def test_scale_zero_gives_mean_of_valid_values():
    B, L, H, D = 2, 6, 2, 4
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=3)
    valid_len = [6, 4]
    out, lse = attention_forward(q, k, v, gains, valid_len, 0.0, 1e-6)
    for b, n in enumerate(valid_len):
        for h in range(H):
            np.testing.assert_allclose(out[b, :, h], np.broadcast_to(v[b, :n, h].mean(0), (L, D)), rtol=1e-13)
            np.testing.assert_allclose(lse[b, h], np.full(L, math.log(n)), rtol=1e-14)


def test_single_token():
    q, k, v, gains, _ = rand_case(1, 1, 2, 4, seed=4)
    scale, eps = 0.9, 1e-6
    out, lse = attention_forward(q, k, v, gains, None, scale, eps)
    np.testing.assert_allclose(out, v, rtol=1e-14)
    for h in range(2):
        qn = q[0, 0, h] / np.sqrt(np.mean(q[0, 0, h] ** 2) + eps) * gains[0]
        kn = k[0, 0, h] / np.sqrt(np.mean(k[0, 0, h] ** 2) + eps) * gains[1]
        assert abs(lse[0, h, 0] - scale * float(qn @ kn)) < 1e-13


def test_no_valid_key_row():
    q, k, v, gains, dout = rand_case(2, 4, 1, 4, seed=5)
    r = attention_fwd_bwd(q, k, v, gains, dout, [0, 4], 0.5, 1e-6)
    assert np.all(r["out"][0] == 0) and np.all(np.isneginf(r["lse"][0]))
    assert np.all(r["dq"][0] == 0) and np.all(r["dk"][0] == 0) and np.all(r["dv"][0] == 0)


# ---------------------------------------------------------------- invariances
def test_softmax_rows_sum_to_one_and_mask():
    q, k, v, gains, _ = rand_case(1, 9, 1, 8, seed=6)
    f = head_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], gains[0], gains[1], 6, 1.3, 1e-6)
    P = f["P"]
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-13)
    assert np.all(P[:, 6:] == 0)


def test_key_permutation_invariance_and_query_equivariance():
    B, L, H, D = 1, 8, 2, 4
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=7)
    n = 6
    base = attention_fwd_bwd(q, k, v, gains, dout, [n], 0.8, 1e-6)
    rng = np.random.default_rng(0)
    perm = np.concatenate([rng.permutation(n), np.arange(n, L)])  # permute valid keys only
    kp, vp = k[:, perm], v[:, perm]
    r = attention_fwd_bwd(q, kp, vp, gains, dout, [n], 0.8, 1e-6)
    np.testing.assert_allclose(r["out"], base["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["lse"], base["lse"], rtol=1e-13)
    np.testing.assert_allclose(r["dk"], base["dk"][:, perm], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dv"], base["dv"][:, perm], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dgains"], base["dgains"], rtol=1e-11, atol=1e-14)
    qperm = rng.permutation(L)
    r = attention_fwd_bwd(q[:, qperm], k, v, gains, dout[:, qperm], [n], 0.8, 1e-6)
    np.testing.assert_allclose(r["out"], base["out"][:, qperm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["lse"], base["lse"][:, :, qperm], rtol=1e-13)
    np.testing.assert_allclose(r["dq"], base["dq"][:, qperm], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dk"], base["dk"], rtol=1e-11, atol=1e-14)


def test_identical_value_rows():
    B, L, H, D = 1, 7, 2, 4
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=8)
    u = np.array([0.5, -1.0, 2.0, 0.25])
    v[:] = u
    r = attention_fwd_bwd(q, k, v, gains, dout, None, 0.6, 1e-6)
    np.testing.assert_allclose(r["out"], np.broadcast_to(u, r["out"].shape), rtol=1e-13)
    assert np.max(np.abs(r["dq"])) < 1e-12
    assert np.max(np.abs(r["dk"])) < 1e-12
    assert np.max(np.abs(r["dgains"])) < 1e-12


def test_rmsnorm_scale_invariance():
    B, L, H, D = 1, 6, 1, 8
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=9)
    eps = 1e-12
    base = attention_fwd_bwd(q, k, v, gains, dout, None, 0.5, eps)
    q2 = q.copy()
    q2[0, 2] *= 7.0
    r = attention_fwd_bwd(q2, k, v, gains, dout, None, 0.5, eps)
    np.testing.assert_allclose(r["out"], base["out"], rtol=1e-9)
    np.testing.assert_allclose(r["dq"][0, 2], base["dq"][0, 2] / 7.0, rtol=1e-8)
    # the gradient of a normalised row is orthogonal to the row
    for i in range(L):
        assert abs(np.dot(base["dq"][0, i, 0], q[0, i, 0])) < 1e-9


def test_gain_identity_and_value_column_sum():
    B, L, H, D = 2, 7, 2, 6
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=10)
    r = attention_fwd_bwd(q, k, v, gains, dout, [7, 5], 0.9, 1e-6)
    # <g_q, dg_q> and <g_k, dg_k> both equal sum_ij dS_ij S_ij (the scores are bilinear in the gains)
    assert abs(np.dot(gains[0], r["dgains"][0]) - np.dot(gains[1], r["dgains"][1])) < 1e-12
    # P rows sum to one, so the value gradients sum to the output gradients
    np.testing.assert_allclose(r["dv"].sum(axis=1), dout.sum(axis=1), rtol=1e-12, atol=1e-13)


def test_padded_keys_do_not_matter():
    B, L, H, D = 2, 8, 2, 4
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=11)
    valid_len = [5, 8]
    base = attention_fwd_bwd(q, k, v, gains, dout, valid_len, 0.7, 1e-6)
    k2, v2 = k.copy(), v.copy()
    k2[0, 5:] = 100.0 * np.random.default_rng(1).standard_normal(k2[0, 5:].shape)
    v2[0, 5:] = -50.0
    r = attention_fwd_bwd(q, k2, v2, gains, dout, valid_len, 0.7, 1e-6)
    for key in ("out", "lse", "dq", "dgains"):
        np.testing.assert_allclose(r[key], base[key], rtol=1e-12, atol=1e-14)
    assert np.all(r["dk"][0, 5:] == 0) and np.all(r["dv"][0, 5:] == 0)
    np.testing.assert_allclose(r["dk"][:, :5], base["dk"][:, :5], rtol=1e-12, atol=1e-14)


def test_valid_len_is_clamped():
    q, k, v, gains, dout = rand_case(2, 5, 1, 4, seed=12)
    a = attention_fwd_bwd(q, k, v, gains, dout, [9, -3], 0.5, 1e-6)
    b = attention_fwd_bwd(q, k, v, gains, dout, [5, 0], 0.5, 1e-6)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_pairs_subset_matches_full():
    q, k, v, gains, dout = rand_case(2, 5, 3, 4, seed=13)
    full = attention_fwd_bwd(q, k, v, gains, dout, None, 0.5, 1e-6)
    sub = attention_fwd_bwd(q, k, v, gains, dout, None, 0.5, 1e-6, pairs=[(1, 2), (0, 0)])
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_array_equal(sub[key][1, :, 2], full[key][1, :, 2])
        assert np.all(np.isnan(sub[key][1, :, 1]))
    np.testing.assert_array_equal(sub["lse"][0, 0], full["lse"][0, 0])
