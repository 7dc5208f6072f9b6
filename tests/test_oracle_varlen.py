"""Pins for the packed variable-length form of the fp64 oracle (sequences of different lengths stored
back to back, each attending only to itself; the variable-length path of the diffusion-pipe summary's
attention wrapper). None re-types the oracle's formulas: finite differences, the reduction to the
(separately pinned) fixed-length and padded forms, and the isolation and ordering properties that a
slicing mistake would break."""
import numpy as np
import pytest

from oracle import attention_fwd_bwd, varlen_fwd_bwd


def rand_packed(lengths, H=2, D=4, seed=0, gain_std=0.3):
    rng = np.random.default_rng(seed)
    total = int(sum(lengths))
    t = lambda: rng.standard_normal((total, H, D))
    q, k, v = t(), t(), t()
    gains = 1.0 + gain_std * rng.standard_normal((2, D))
    dout = t()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(int)
    return q, k, v, gains, dout, cu


def loss(q, k, v, gains, dout, cu, scale, eps):
    r = varlen_fwd_bwd(q, k, v, gains, dout, cu, scale, eps)
    return float(np.sum(r["out"] * dout))


def test_finite_difference_gradients():
    """Every element of q, k, v and both gains, on a pack with an empty sequence in the middle."""
    q, k, v, gains, dout, cu = rand_packed([3, 0, 4, 2], seed=1)
    scale, eps = 0.7, 1e-3
    r = varlen_fwd_bwd(q, k, v, gains, dout, cu, scale, eps)
    h = 1e-6
    for name, x, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"]), ("gains", gains, r["dgains"])):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v, gains, dout, cu, scale, eps)
            x[idx] = old - h
            lm = loss(q, k, v, gains, dout, cu, scale, eps)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


def test_equal_lengths_are_the_fixed_length_batch():
    B, L, H, D = 3, 5, 2, 4
    q, k, v, gains, dout, cu = rand_packed([L] * B, H, D, seed=2)
    r = varlen_fwd_bwd(q, k, v, gains, dout, cu, 0.6, 1e-6)
    fx = lambda t: t.reshape(B, L, H, D)
    j = attention_fwd_bwd(fx(q), fx(k), fx(v), gains, fx(dout), None, 0.6, 1e-6)
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_allclose(fx(r[key]), j[key], rtol=1e-12, atol=1e-14)
    for b in range(B):
        np.testing.assert_allclose(r["lse"][b], j["lse"][b], rtol=1e-13)
    np.testing.assert_allclose(r["dgains"], j["dgains"], rtol=1e-11, atol=1e-13)


def test_padded_batch_with_key_mask():
    """The same sequences padded to the longest one, keys masked by valid_len and dout zero on the
    padded rows: every result on the real rows, and the gain gradients, are those of the pack."""
    lengths = [6, 2, 5]
    H, D = 2, 4
    q, k, v, gains, dout, cu = rand_packed(lengths, H, D, seed=3)
    r = varlen_fwd_bwd(q, k, v, gains, dout, cu, 0.8, 1e-6)
    B, Lm = len(lengths), max(lengths)
    rng = np.random.default_rng(7)
    pad = lambda t: np.stack([np.concatenate([t[cu[b]:cu[b + 1]], rng.standard_normal((Lm - lengths[b], H, D))])
                              for b in range(B)])
    dpad = np.stack([np.concatenate([dout[cu[b]:cu[b + 1]], np.zeros((Lm - lengths[b], H, D))]) for b in range(B)])
    j = attention_fwd_bwd(pad(q), pad(k), pad(v), gains, dpad, lengths, 0.8, 1e-6)
    for b, n in enumerate(lengths):
        for key in ("out", "dq", "dk", "dv"):
            np.testing.assert_allclose(r[key][cu[b]:cu[b + 1]], j[key][b, :n], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(r["lse"][b], j["lse"][b, :, :n], rtol=1e-13)
    np.testing.assert_allclose(r["dgains"], j["dgains"], rtol=1e-11, atol=1e-13)


def test_sequences_are_isolated():
    q, k, v, gains, dout, cu = rand_packed([4, 3, 5], seed=4)
    base = varlen_fwd_bwd(q, k, v, gains, dout, cu, 0.5, 1e-6)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] *= -3.0
    v2[cu[1]:cu[2]] += 10.0
    r = varlen_fwd_bwd(q, k2, v2, gains, dout, cu, 0.5, 1e-6)
    for b in (0, 2):
        sl = slice(cu[b], cu[b + 1])
        for key in ("out", "dq", "dk", "dv"):
            np.testing.assert_array_equal(r[key][sl], base[key][sl])
        np.testing.assert_array_equal(r["lse"][b], base["lse"][b])
    assert not np.allclose(r["out"][cu[1]:cu[2]], base["out"][cu[1]:cu[2]])


def test_reordering_sequences_permutes_results():
    lengths = [4, 1, 6, 3]
    q, k, v, gains, dout, cu = rand_packed(lengths, seed=5)
    base = varlen_fwd_bwd(q, k, v, gains, dout, cu, 0.9, 1e-6)
    order = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    cu2 = np.concatenate([[0], np.cumsum([lengths[b] for b in order])])
    r = varlen_fwd_bwd(q[rows], k[rows], v[rows], gains, dout[rows], cu2, 0.9, 1e-6)
    for key in ("out", "dq", "dk", "dv"):
        np.testing.assert_allclose(r[key], base[key][rows], rtol=1e-12, atol=1e-14)
    for i, b in enumerate(order):
        np.testing.assert_allclose(r["lse"][i], base["lse"][b], rtol=1e-13)
    np.testing.assert_allclose(r["dgains"], base["dgains"], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seqs", [[1], [0, 2]])
def test_sequence_subset(seqs):
    q, k, v, gains, dout, cu = rand_packed([3, 4, 2], seed=6)
    full = varlen_fwd_bwd(q, k, v, gains, dout, cu, 0.5, 1e-6)
    sub = varlen_fwd_bwd(q, k, v, gains, dout, cu, 0.5, 1e-6, seqs=seqs)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        if b in seqs:
            np.testing.assert_array_equal(sub["out"][sl], full["out"][sl])
        else:
            assert np.all(np.isnan(sub["out"][sl])) and sub["lse"][b] is None
