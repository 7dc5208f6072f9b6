"""Pins for the fp64 oracle of the adaLN-modulated QKV projection (LayerNorm without affine, per-sample
scale and shift, then a linear layer C -> 3C with bias, split into q, k, v heads). None re-types the
oracle's formulas: finite differences of every input, torch's fp64 layer_norm and linear with
autograd as independent routines, closed forms for special weights and modulations, and the
invariances of a LayerNorm that a dropped term or a wrong axis would break."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import adaln_qkv_backward, adaln_qkv_forward, adaln_qkv_fwd_bwd


def rand_case(B=2, N=3, C=8, H=2, seed=0, mod_std=0.4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, C)) * 1.5 + 0.3
    mod = mod_std * rng.standard_normal((B, 2, C))
    w = rng.standard_normal((3 * C, C)) / np.sqrt(C)
    bias = 0.2 * rng.standard_normal(3 * C)
    D = C // H
    dq, dk, dv = (rng.standard_normal((B, N, H, D)) for _ in range(3))
    return x, mod, w, bias, dq, dk, dv


def loss(x, mod, w, bias, H, eps, dq, dk, dv):
    f = adaln_qkv_forward(x, mod, w, bias, H, eps)
    return float(np.sum(f["q"] * dq) + np.sum(f["k"] * dk) + np.sum(f["v"] * dv))


@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_finite_difference_gradients(eps):
    x, mod, w, bias, dq, dk, dv = rand_case(seed=1)
    H = 2
    g = adaln_qkv_backward(x, mod, w, bias, H, eps, dq, dk, dv)
    h = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("mod", mod, g["dmod"]), ("w", w, g["dw"]), ("bias", bias, g["dbias"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(x, mod, w, bias, H, eps, dq, dk, dv)
            arr[idx] = old - h
            lm = loss(x, mod, w, bias, H, eps, dq, dk, dv)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-6, (name, eps, err)


def test_matches_torch_layer_norm_and_linear_fp64():
    B, N, C, H = 2, 5, 16, 4
    x, mod, w, bias, dq, dk, dv = rand_case(B, N, C, H, seed=2)
    eps = 1e-6
    got = adaln_qkv_fwd_bwd(x, mod, w, bias, H, eps, dq, dk, dv)
    tx, tm, tw, tb = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, mod, w, bias))
    hh = F.layer_norm(tx, (C,), eps=eps) * (1 + tm[:, 1:2]) + tm[:, 0:1]
    y = F.linear(hh, tw, tb)
    q, k, v = (t.reshape(B, N, H, C // H) for t in y.split(C, dim=-1))
    (q * torch.tensor(dq)).sum().add((k * torch.tensor(dk)).sum()).add((v * torch.tensor(dv)).sum()).backward()
    for key, t in (("q", q), ("k", k), ("v", v), ("h", hh)):
        np.testing.assert_allclose(got[key], t.detach().numpy(), rtol=1e-12, atol=1e-13)
    for key, t in (("dx", tx), ("dmod", tm), ("dw", tw), ("dbias", tb)):
        np.testing.assert_allclose(got[key], t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_identity_weights_give_the_modulated_rows():
    """w = [I; I; I], no bias: q = k = v = h, and with scale = shift = 0 each row of h has mean 0 and
    mean square var / (var + eps) (worked by hand from the row's own values)."""
    B, N, C, H = 1, 4, 8, 2
    rng = np.random.default_rng(3)
    x = rng.standard_normal((B, N, C)) * 2.0 + 1.0
    w = np.concatenate([np.eye(C)] * 3)
    eps = 1e-2
    f = adaln_qkv_forward(x, np.zeros((B, 2, C)), w, None, H, eps)
    for key in ("q", "k", "v"):
        np.testing.assert_allclose(f[key].reshape(B, N, C), f["h"], rtol=1e-14, atol=1e-15)
    for i in range(N):
        row = x[0, i]
        m = sum(row) / C
        var = sum((t - m) ** 2 for t in row) / C
        np.testing.assert_allclose(f["h"][0, i].mean(), 0.0, atol=1e-14)
        np.testing.assert_allclose(np.mean(f["h"][0, i] ** 2), var / (var + eps), rtol=1e-13)
        np.testing.assert_allclose(f["mean"][0, i], m, rtol=1e-13)
        np.testing.assert_allclose(f["rstd"][0, i], 1.0 / np.sqrt(var + eps), rtol=1e-13)


def test_modulation_closed_form():
    """With w = [I; I; I] the output equals LN(x) * (1 + scale_b) + shift_b channel by channel, so
    shift alone moves q by shift and scale = -1 leaves exactly shift."""
    B, N, C, H = 2, 3, 4, 1
    x, mod, _, _, _, _, _ = rand_case(B, N, C, H, seed=4)
    w = np.concatenate([np.eye(C)] * 3)
    base = adaln_qkv_forward(x, np.zeros_like(mod), w, None, H, 1e-6)["q"].reshape(B, N, C)
    m2 = mod.copy()
    m2[:, 1] = 0.0
    shifted = adaln_qkv_forward(x, m2, w, None, H, 1e-6)["q"].reshape(B, N, C)
    np.testing.assert_allclose(shifted - base, np.broadcast_to(mod[:, 0][:, None, :], (B, N, C)), atol=1e-13)
    m3 = mod.copy()
    m3[:, 1] = -1.0
    killed = adaln_qkv_forward(x, m3, w, None, H, 1e-6)["q"].reshape(B, N, C)
    np.testing.assert_allclose(killed, np.broadcast_to(mod[:, 0][:, None, :], (B, N, C)), atol=1e-15)


def test_row_affine_invariance():
    """LayerNorm ignores a per-row positive scale and offset of its input (up to eps): q, k, v stay,
    and dx scales by 1/a."""
    x, mod, w, bias, dq, dk, dv = rand_case(seed=5)
    a = np.array([2.0, 0.5])[:, None, None] * np.array([1.0, 3.0, 0.25])[None, :, None]
    c = np.array([5.0, -1.0])[:, None, None]
    r1 = adaln_qkv_fwd_bwd(x, mod, w, bias, 2, 0.0, dq, dk, dv)
    r2 = adaln_qkv_fwd_bwd(a * x + c, mod, w, bias, 2, 0.0, dq, dk, dv)
    for key in ("q", "k", "v"):
        np.testing.assert_allclose(r2[key], r1[key], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r2["dx"] * a, r1["dx"], rtol=1e-9, atol=1e-11)
    for key in ("dmod", "dw", "dbias"):
        np.testing.assert_allclose(r2[key], r1[key], rtol=1e-10, atol=1e-12)


def test_input_gradient_is_orthogonal_to_ones_and_xhat():
    """Adding a constant to a row, or stretching it about its mean, changes nothing (eps = 0), so dx
    of every row is orthogonal to the all-ones vector and to xhat."""
    x, mod, w, bias, dq, dk, dv = rand_case(B=3, N=4, C=12, H=3, seed=6)
    r = adaln_qkv_fwd_bwd(x, mod, w, bias, 3, 0.0, dq, dk, dv)
    assert np.max(np.abs(r["dx"].sum(axis=-1))) < 1e-12
    assert np.max(np.abs((r["dx"] * r["xhat"]).sum(axis=-1))) < 1e-12


def test_samples_are_isolated_and_bias_gradient_counts_every_token():
    x, mod, w, bias, dq, dk, dv = rand_case(B=3, N=2, C=8, H=2, seed=7)
    base = adaln_qkv_fwd_bwd(x, mod, w, bias, 2, 1e-6, dq, dk, dv)
    m2 = mod.copy()
    m2[1] *= -2.0
    r = adaln_qkv_fwd_bwd(x, m2, w, bias, 2, 1e-6, dq, dk, dv)
    for b in (0, 2):
        for key in ("q", "k", "v", "dx"):
            np.testing.assert_array_equal(r[key][b], base[key][b])
        np.testing.assert_array_equal(r["dmod"][b], base["dmod"][b])
    assert not np.allclose(r["q"][1], base["q"][1])
    # zero weights: the outputs are the bias on every token, and nothing reaches x or mod
    z = adaln_qkv_fwd_bwd(x, mod, np.zeros_like(w), bias, 2, 1e-6, dq, dk, dv)
    np.testing.assert_array_equal(z["q"], np.broadcast_to(bias[:8].reshape(2, 4), z["q"].shape))
    assert np.all(z["dx"] == 0) and np.all(z["dmod"] == 0)
    # the bias gradient is the upstream gradient summed over all 6 tokens, column by column
    cols = np.concatenate([t.reshape(6, 8) for t in (dq, dk, dv)], axis=1)
    np.testing.assert_allclose(z["dbias"], [sum(cols[i, j] for i in range(6)) for j in range(24)], rtol=1e-13)


def test_scale_minus_one_cuts_x_off():
    """scale = -1 on every channel makes h = shift whatever x is: dx is exactly zero, while the
    modulation and weight gradients are not."""
    x, mod, w, bias, dq, dk, dv = rand_case(seed=8)
    mod[:, 1] = -1.0
    r = adaln_qkv_fwd_bwd(x, mod, w, bias, 2, 1e-6, dq, dk, dv)
    assert np.all(r["dx"] == 0)
    assert np.max(np.abs(r["dmod"][:, 1])) > 1e-3 and np.max(np.abs(r["dw"])) > 1e-3


def test_euler_identities_of_the_linear_parameters():
    """The loss is linear in (w, bias) jointly, affine in shift and affine in (1 + scale), so each
    gradient contracted with its own parameter gives the part of the loss that parameter carries."""
    x, mod, w, bias, dq, dk, dv = rand_case(B=2, N=4, C=8, H=2, seed=9)
    L = lambda m=mod, ww=w, bb=bias: loss(x, m, ww, bb, 2, 1e-6, dq, dk, dv)
    r = adaln_qkv_backward(x, mod, w, bias, 2, 1e-6, dq, dk, dv)
    np.testing.assert_allclose(np.sum(r["dw"] * w) + np.sum(r["dbias"] * bias), L(), rtol=1e-12)
    no_shift = mod.copy()
    no_shift[:, 0] = 0.0
    np.testing.assert_allclose(np.sum(r["dmod"][:, 0] * mod[:, 0]), L() - L(m=no_shift), rtol=1e-11)
    cut = mod.copy()
    cut[:, 1] = -1.0
    np.testing.assert_allclose(np.sum(r["dmod"][:, 1] * (1.0 + mod[:, 1])), L() - L(m=cut), rtol=1e-11)
