"""Pins for the fp64 oracle of the per-stream MLP block (fc, adaLN, SwiGLU, one residual). None re-types
the oracle's formulas: finite differences of every input, torch's fp64 linear, layer_norm and silu with
autograd, a closed form worked element by element with math.exp, and identities that follow from the
block's linearity in some of its parameters."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mlp_backward, mlp_forward, mlp_fwd_bwd


def rand_case(B=2, N=2, C=4, Fh=3, seed=0):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s)
    return dict(o=r(B, N, C), x=r(B, N, C), mod=0.4 * r(B, 2, C), wfc=r(C, C) / math.sqrt(C), bfc=0.2 * r(C),
                w12=r(2 * Fh, C) / math.sqrt(C), b12=0.2 * r(2 * Fh), w2=r(C, Fh) / math.sqrt(Fh), b2=0.2 * r(C),
                dout=r(B, N, C))


ARGS = ("o", "x", "mod", "wfc", "bfc", "w12", "b12", "w2", "b2")


def loss(c, eps):
    out = mlp_forward(*(c[k] for k in ARGS), eps)["out"]
    return float(np.sum(out * c["dout"]))


@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_finite_difference_gradients(eps):
    c = rand_case(seed=1)
    g = mlp_backward(*(c[k] for k in ARGS), eps, c["dout"])
    h = 1e-6
    for name in ARGS:
        arr, grad = c[name], g["d" + name]
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(c, eps)
            arr[idx] = old - h
            lm = loss(c, eps)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-6, (name, eps, err)


def test_matches_torch_fp64_autograd():
    c = rand_case(B=2, N=5, C=8, Fh=12, seed=2)
    eps = 1e-6
    got = mlp_fwd_bwd(*(c[k] for k in ARGS), eps, c["dout"])
    t = {k: torch.tensor(c[k], dtype=torch.float64, requires_grad=True) for k in ARGS}
    z = F.linear(t["o"], t["wfc"], t["bfc"])
    u = F.layer_norm(z, (8,), eps=eps) * (1 + t["mod"][:, 1:2]) + t["mod"][:, 0:1]
    a, g = F.linear(u, t["w12"], t["b12"]).chunk(2, dim=-1)
    out = t["x"] + F.linear(F.silu(a) * g, t["w2"], t["b2"])
    (out * torch.tensor(c["dout"])).sum().backward()
    np.testing.assert_allclose(got["out"], out.detach().numpy(), rtol=1e-12, atol=1e-13)
    for k in ARGS:
        np.testing.assert_allclose(got["d" + k], t[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_silu_closed_form():
    """W1 = I, b1 = 0, W3 = 0, b3 = 1, W2 = I, b2 = 0: out = x + silu(u) elementwise, worked with math.exp."""
    c = rand_case(B=1, N=3, C=4, Fh=4, seed=3)
    C = 4
    c["w12"] = np.concatenate([np.eye(C), np.zeros((C, C))])
    c["b12"] = np.concatenate([np.zeros(C), np.ones(C)])
    c["w2"], c["b2"] = np.eye(C), np.zeros(C)
    f = mlp_forward(*(c[k] for k in ARGS), 1e-6)
    for idx in np.ndindex(f["u"].shape):
        uu = f["u"][idx]
        assert abs(f["out"][idx] - (c["x"][idx] + uu / (1.0 + math.exp(-uu)))) < 1e-13


def test_zero_down_projection_is_the_residual():
    c = rand_case(seed=4)
    c["w2"] = np.zeros_like(c["w2"])
    c["b2"] = np.zeros_like(c["b2"])
    r = mlp_fwd_bwd(*(c[k] for k in ARGS), 1e-6, c["dout"])
    np.testing.assert_array_equal(r["out"], c["x"])
    np.testing.assert_array_equal(r["dx"], c["dout"])
    for k in ("do", "dmod", "dwfc", "dbfc", "dw12", "db12"):
        assert np.all(r[k] == 0), k
    assert np.max(np.abs(r["dw2"])) > 1e-3


def test_euler_identities():
    """The loss is linear in (W2, b2) jointly and in the gate half (W3, b3) jointly: each gradient
    contracted with its parameter gives the part of the loss that parameter carries."""
    c = rand_case(B=2, N=3, C=6, Fh=5, seed=5)
    r = mlp_fwd_bwd(*(c[k] for k in ARGS), 1e-6, c["dout"])
    Fh = 5
    Ly = float(np.sum(c["dout"] * r["y"]))
    np.testing.assert_allclose(np.sum(r["dw2"] * c["w2"]) + np.sum(r["db2"] * c["b2"]), Ly, rtol=1e-12)
    gate = np.sum(r["dw12"][Fh:] * c["w12"][Fh:]) + np.sum(r["db12"][Fh:] * c["b12"][Fh:])
    np.testing.assert_allclose(gate, Ly - float(np.sum(c["dout"] * c["b2"])), rtol=1e-11)


def test_samples_are_isolated():
    c = rand_case(B=3, N=2, C=4, Fh=3, seed=6)
    base = mlp_fwd_bwd(*(c[k] for k in ARGS), 1e-6, c["dout"])
    c2 = {k: v.copy() for k, v in c.items()}
    c2["mod"][1] *= -3.0
    c2["o"][1] += 1.0
    r = mlp_fwd_bwd(*(c2[k] for k in ARGS), 1e-6, c2["dout"])
    for b in (0, 2):
        for k in ("out", "do", "dx"):
            np.testing.assert_array_equal(r[k][b], base[k][b])
        np.testing.assert_array_equal(r["dmod"][b], base["dmod"][b])
    assert not np.allclose(r["out"][1], base["out"][1])


def test_silu_derivative_closed_form():
    """In the closed-form set-up (W1 = I, b1 = 0, W3 = 0, b3 = 1, W2 = I) the gradient reaching the
    first half of the gate/up output is dout * silu'(u), silu'(u) = s + u s (1 - s), s = 1 / (1 + e^-u)."""
    c = rand_case(B=1, N=3, C=4, Fh=4, seed=7)
    C = 4
    c["w12"] = np.concatenate([np.eye(C), np.zeros((C, C))])
    c["b12"] = np.concatenate([np.zeros(C), np.ones(C)])
    c["w2"], c["b2"] = np.eye(C), np.zeros(C)
    r = mlp_fwd_bwd(*(c[k] for k in ARGS), 1e-6, c["dout"])
    for idx in np.ndindex(r["u"].shape):
        uu = r["u"][idx]
        s = 1.0 / (1.0 + math.exp(-uu))
        assert abs(r["dag"][idx] - c["dout"][idx] * (s + uu * s * (1.0 - s))) < 1e-13


def test_layer_norm_scale_invariance_identities():
    """With eps = 0 the LayerNorm ignores a common scale of its input z = o Wfc^T + bfc: scaling (Wfc, bfc)
    together, or (o, bfc) together, changes nothing, so <dWfc, Wfc> + <dbfc, bfc> = 0 and
    <do, o> + <dbfc, bfc> = 0."""
    c = rand_case(B=2, N=3, C=6, Fh=5, seed=8)
    r = mlp_fwd_bwd(*(c[k] for k in ARGS), 0.0, c["dout"])
    scale_ref = np.sum(np.abs(r["dwfc"] * c["wfc"])) + np.sum(np.abs(r["dbfc"] * c["bfc"]))
    assert abs(np.sum(r["dwfc"] * c["wfc"]) + np.sum(r["dbfc"] * c["bfc"])) < 1e-12 * max(1.0, scale_ref)
    assert abs(np.sum(r["do"] * c["o"]) + np.sum(r["dbfc"] * c["bfc"])) < 1e-12 * max(1.0, scale_ref)


def test_constant_gate_modulation_identities():
    """W1 = 0 and b1 = 3 make silu(a) the constant silu(3): the block is then linear in the modulated input
    u, so the loss is affine in shift and in (1 + scale), and <dshift, shift> = L - L(shift = 0),
    <dscale, 1 + scale> = L - L(scale = -1)."""
    c = rand_case(B=2, N=3, C=5, Fh=4, seed=9)
    c["w12"][:4] = 0.0
    c["b12"][:4] = 3.0
    L = lambda m: float(np.sum(c["dout"] * mlp_forward(c["o"], c["x"], m, *(c[k] for k in ARGS[3:]), 1e-6)["out"]))
    r = mlp_fwd_bwd(*(c[k] for k in ARGS), 1e-6, c["dout"])
    no_shift = c["mod"].copy()
    no_shift[:, 0] = 0.0
    cut = c["mod"].copy()
    cut[:, 1] = -1.0
    np.testing.assert_allclose(np.sum(r["dmod"][:, 0] * c["mod"][:, 0]), L(c["mod"]) - L(no_shift), rtol=1e-10)
    np.testing.assert_allclose(np.sum(r["dmod"][:, 1] * (1 + c["mod"][:, 1])), L(c["mod"]) - L(cut), rtol=1e-10)


def test_scale_minus_one_cuts_the_attention_output_off():
    """scale = -1 makes the modulated input the shift alone: nothing before the LayerNorm matters, so do,
    dWfc and dbfc are exactly zero."""
    c = rand_case(seed=10)
    c["mod"][:, 1] = -1.0
    r = mlp_fwd_bwd(*(c[k] for k in ARGS), 1e-6, c["dout"])
    for k in ("do", "dwfc", "dbfc"):
        assert np.all(r[k] == 0), k
    assert np.max(np.abs(r["dw12"])) > 1e-3
