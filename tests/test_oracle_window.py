"""Pins for the local-window option of the fp64 oracle (the windowed attention of the diffusion-pipe
summary's attention wrapper, read as a sliding window: query i sees keys i - left .. i + right).
Independent of the oracle's formulas: finite differences, the closed form of a zero-width window,
the unwindowed oracle restricted to each row's keys (brute force per row), the token-reversal symmetry
that exchanges the two bounds, and torch's fp64 causal scaled_dot_product_attention with autograd for
the windows (-1, 0) and, on reversed tokens, (0, -1)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_forward, attention_fwd_bwd


def rand_case(B=2, L=7, H=2, D=4, seed=0, gain_std=0.3):
    rng = np.random.default_rng(seed)
    t = lambda: rng.standard_normal((B, L, H, D))
    q, k, v = t(), t(), t()
    gains = 1.0 + gain_std * rng.standard_normal((2, D))
    return q, k, v, gains, t()


@pytest.mark.parametrize("window,valid_len", [((2, 1), None), ((1, 3), [7, 5]), ((0, 2), [7, 3])])
def test_finite_difference_gradients(window, valid_len):
    q, k, v, gains, dout = rand_case(seed=1)
    scale, eps = 0.7, 1e-3
    r = attention_fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps, window=window)
    loss = lambda: float(np.sum(attention_forward(q, k, v, gains, valid_len, scale, eps, window=window)[0] * dout))
    h = 1e-6
    for name, x, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"]), ("gains", gains, r["dgains"])):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("window", [(-1, -1), (7, 7), (100, -1)])
def test_unbounded_window_is_no_window(window):
    q, k, v, gains, dout = rand_case(seed=2)
    a = attention_fwd_bwd(q, k, v, gains, dout, [7, 4], 0.6, 1e-6, window=window)
    b = attention_fwd_bwd(q, k, v, gains, dout, [7, 4], 0.6, 1e-6)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-14)


def test_zero_width_window():
    """Each query sees only its own key: O_i = v_i and LSE_i = scale <Qn_i, Kn_i> for i < n; rows at
    or past n see nothing (O = 0, LSE = -inf)."""
    q, k, v, gains, dout = rand_case(B=1, L=6, H=1, D=4, seed=3)
    scale, eps, n = 0.8, 1e-6, 4
    r = attention_fwd_bwd(q, k, v, gains, dout, [n], scale, eps, window=(0, 0))
    np.testing.assert_allclose(r["out"][0, :n], v[0, :n], rtol=1e-13)
    assert np.all(r["out"][0, n:] == 0) and np.all(np.isneginf(r["lse"][0, 0, n:]))
    for i in range(n):
        qn = q[0, i, 0] / np.sqrt(np.mean(q[0, i, 0] ** 2) + eps) * gains[0]
        kn = k[0, i, 0] / np.sqrt(np.mean(k[0, i, 0] ** 2) + eps) * gains[1]
        assert abs(r["lse"][0, 0, i] - scale * float(qn @ kn)) < 1e-12
    # with one key per row the softmax is constant: no gradient reaches q or k
    assert np.max(np.abs(r["dq"])) < 1e-12 and np.max(np.abs(r["dk"])) < 1e-12


@pytest.mark.parametrize("window", [(2, 1), (0, 3), (4, 0)])
def test_each_row_is_attention_over_its_window(window):
    """Row i of the windowed result = row i of the unwindowed attention computed over only the keys
    max(0, i - left) .. min(n, i + right + 1) - 1 (brute force: one small attention per row)."""
    B, L, H, D = 1, 9, 2, 4
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=4)
    n = 8
    r = attention_forward(q, k, v, gains, [n], 0.9, 1e-6, window=window)
    left, right = window
    for i in range(L):
        lo, hi = max(0, i - left), min(n, i + right + 1)
        if hi <= lo:
            assert np.all(r[0][0, i] == 0) and np.all(np.isneginf(r[1][0, :, i]))
            continue
        # the query row followed by its window's keys; only row 0 of this small problem is used
        qs = np.concatenate([q[:, i:i + 1], np.zeros((B, hi - lo - 1, H, D))], axis=1) if hi - lo > 1 else q[:, i:i + 1]
        o, lse = attention_forward(qs, k[:, lo:hi], v[:, lo:hi], gains, None, 0.9, 1e-6)
        np.testing.assert_allclose(r[0][0, i], o[0, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r[1][0, :, i], lse[0, :, 0], rtol=1e-12)


@pytest.mark.parametrize("window", [(4, 1), (0, 2), (3, 0)])
def test_reversing_tokens_swaps_left_and_right(window):
    """With every key valid, reading the sequence backwards turns the window (a, b) into (b, a): the
    results on the reversed tokens are the reversed results, and the gain gradients are unchanged."""
    q, k, v, gains, dout = rand_case(B=2, L=8, H=2, D=4, seed=6)
    a = attention_fwd_bwd(q, k, v, gains, dout, None, 0.7, 1e-6, window=window)
    rev = lambda t: t[:, ::-1].copy()
    b = attention_fwd_bwd(rev(q), rev(k), rev(v), gains, rev(dout), None, 0.7, 1e-6, window=window[::-1])
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_allclose(rev(b[key]), a[key], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(b["lse"][:, :, ::-1], a["lse"], rtol=1e-13)
    np.testing.assert_allclose(b["dgains"], a["dgains"], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("window", [(-1, 0), (0, -1)])
def test_causal_window_matches_torch_sdpa_fp64(window):
    """(-1, 0) is torch's causal attention; (0, -1), each query seeing itself and the keys after it, is
    torch's causal attention on the token-reversed inputs, reversed back."""
    B, L, H, D = 2, 7, 3, 8
    q, k, v, gains, dout = rand_case(B, L, H, D, seed=5)
    scale, eps = 0.4, 1e-6
    got = attention_fwd_bwd(q, k, v, gains, dout, None, scale, eps, window=window)
    if window == (0, -1):
        q, k, v, dout = (t[:, ::-1].copy() for t in (q, k, v, dout))
        got = {key: (val[:, ::-1] if key in ("out", "dq", "dk", "dv") else val) for key, val in got.items()}
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tg = torch.tensor(gains, dtype=torch.float64, requires_grad=True)
    nq = F.rms_norm(tq, (D,), weight=tg[0], eps=eps)
    nk = F.rms_norm(tk, (D,), weight=tg[1], eps=eps)
    Q, K, V = (t.permute(0, 2, 1, 3) for t in (nq, nk, tv))
    O = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale).permute(0, 2, 1, 3)
    O.backward(torch.tensor(dout))
    np.testing.assert_allclose(got["out"], O.detach().numpy(), rtol=1e-10, atol=1e-12)
    for key, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dgains", tg)):
        np.testing.assert_allclose(got[key], t.grad.numpy(), rtol=1e-9, atol=1e-11)
