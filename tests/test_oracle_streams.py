"""Pins for the two-stream form of the fp64 oracle (image and text tokens in separate tensors, each
stream with its own QK-norm gains; re-diffusion README, the DiT-layer box of the architecture
flowchart: QKV per stream, concat, joint attention, split). As for the joint form, none of these
re-types the oracle's formulas: finite differences, a closed form worked by hand, the reduction to
the (separately pinned) joint oracle when both streams share their gains, and the symmetry under
swapping the roles of the two streams."""
import math

import numpy as np
import pytest

from oracle import attention_fwd_bwd, streams_fwd_bwd


def rand_streams(B=2, n_img=3, n_txt=2, H=2, D=4, seed=0, gain_std=0.3):
    rng = np.random.default_rng(seed)
    pair = lambda: (rng.standard_normal((B, n_img, H, D)), rng.standard_normal((B, n_txt, H, D)))
    q, k, v = pair(), pair(), pair()
    gains = 1.0 + gain_std * rng.standard_normal((2, 2, D))
    dout = pair()
    return q, k, v, gains, dout


def loss(q, k, v, gains, dout, valid_len, scale, eps):
    r = streams_fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps)
    return float(sum(np.sum(o * d) for o, d in zip(r["out"], dout)))


@pytest.mark.parametrize("valid_len", [None, [5, 4], [2, 5]])
def test_finite_difference_gradients(valid_len):
    """Every element of both streams of q, k, v and of all four gain vectors. valid_len [5, 4] pads
    the last text key of sequence 1; [2, 5] leaves sequence 0 with image keys only."""
    q, k, v, gains, dout = rand_streams(seed=1)
    scale, eps = 0.7, 1e-3
    r = streams_fwd_bwd(q, k, v, gains, dout, valid_len, scale, eps)
    h = 1e-6
    cases = [(f"{name}[{s}]", t[s], r[name][s]) for name, t in (("dq", q), ("dk", k), ("dv", v)) for s in (0, 1)]
    cases.append(("dgains", gains, r["dgains"]))
    for name, x, grad in cases:
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


def test_closed_form_distinct_stream_gains():
    """D = 1, eps = 0: the RMSNorm of a scalar is sign(x) * g. One image token (q = 1, k = 3) with
    gains (g_q, g_k) = (2, 1.5) and one text token (q = -2, k = -0.5) with gains (0.5, -1); scale 0.5.
    Scores by hand: row 0 (image query) = 0.5 * 2 * (1.5, 1) = (1.5, 1.0); row 1 (text query) =
    0.5 * -0.5 * (1.5, 1) = (-0.375, -0.25). Each row is a two-term softmax."""
    q = (np.array([1.0]).reshape(1, 1, 1, 1), np.array([-2.0]).reshape(1, 1, 1, 1))
    k = (np.array([3.0]).reshape(1, 1, 1, 1), np.array([-0.5]).reshape(1, 1, 1, 1))
    v = (np.array([0.7]).reshape(1, 1, 1, 1), np.array([-1.1]).reshape(1, 1, 1, 1))
    gains = np.array([[[2.0], [1.5]], [[0.5], [-1.0]]])
    dout = (np.ones((1, 1, 1, 1)), np.ones((1, 1, 1, 1)))
    r = streams_fwd_bwd(q, k, v, gains, dout, None, 0.5, 0.0)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    np.testing.assert_allclose(r["out"][0].ravel(), [sig(0.5) * 0.7 + sig(-0.5) * -1.1], rtol=1e-14)
    np.testing.assert_allclose(r["out"][1].ravel(), [sig(-0.125) * 0.7 + sig(0.125) * -1.1], rtol=1e-14)
    np.testing.assert_allclose(r["lse"].ravel(), [1.5 + math.log1p(math.exp(-0.5)),
                                                  -0.25 + math.log1p(math.exp(-0.125))], rtol=1e-14)


@pytest.mark.parametrize("valid_len", [None, [7, 4]])
def test_shared_gains_reduce_to_joint_form(valid_len):
    """Both streams with the same gains: the joint attention on the concatenated tensors (image
    first), with the per-stream gain gradients summing to the joint ones."""
    q, k, v, gains, dout = rand_streams(B=2, n_img=4, n_txt=3, H=2, D=6, seed=2)
    gains[1] = gains[0]
    r = streams_fwd_bwd(q, k, v, gains, dout, valid_len, 0.6, 1e-6)
    cat = lambda t: np.concatenate(t, axis=1)
    j = attention_fwd_bwd(cat(q), cat(k), cat(v), gains[0], cat(dout), valid_len, 0.6, 1e-6)
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_allclose(cat(r[key]), j[key], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["lse"], j["lse"], rtol=1e-13)
    np.testing.assert_allclose(r["dgains"][0] + r["dgains"][1], j["dgains"], rtol=1e-11, atol=1e-13)


def test_swapping_stream_roles():
    """Giving the text tensors and gains the image role (and vice versa) permutes the joint rows: with
    no key padding, every per-token result follows its tokens and the gain gradients swap streams."""
    q, k, v, gains, dout = rand_streams(B=2, n_img=4, n_txt=3, H=2, D=4, seed=3)
    sw = lambda t: (t[1], t[0])
    a = streams_fwd_bwd(q, k, v, gains, dout, None, 0.8, 1e-6)
    b = streams_fwd_bwd(sw(q), sw(k), sw(v), gains[::-1].copy(), sw(dout), None, 0.8, 1e-6)
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_allclose(b[key][0], a[key][1], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(b[key][1], a[key][0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["lse"], np.concatenate([a["lse"][:, :, 4:], a["lse"][:, :, :4]], axis=2),
                               rtol=1e-13)
    np.testing.assert_allclose(b["dgains"], a["dgains"][::-1], rtol=1e-11, atol=1e-14)


def test_one_stream_empty():
    """No text tokens: the image stream alone is the joint attention with its own gains, and the
    (empty) text stream gets zero gain gradients."""
    q, k, v, gains, dout = rand_streams(B=1, n_img=5, n_txt=0, H=2, D=4, seed=4)
    r = streams_fwd_bwd(q, k, v, gains, dout, [3], 0.5, 1e-6)
    j = attention_fwd_bwd(q[0], k[0], v[0], gains[0], dout[0], [3], 0.5, 1e-6)
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_allclose(r[key][0], j[key], rtol=1e-12, atol=1e-14)
        assert r[key][1].shape == (1, 0, 2, 4)
    np.testing.assert_allclose(r["dgains"][0], j["dgains"], rtol=1e-11, atol=1e-14)
    assert np.all(r["dgains"][1] == 0)
