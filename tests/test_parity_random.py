"""Randomised GPU parity sweep over every entry point family, against the fp64 oracle.

The hand-picked shapes of the other parity files cover known edges; this file draws further
combinations (batch, length or stream split, head count, head dim, key mask, window, widths) from a
fixed list of seeds, so the cases are the same on every run and each prints its parameters before it
runs. Tolerances and comparisons are those of the family's own parity file (imported from it); where
a drawn key mask or window can leave a row with a single key, that row's LSE is one score with no
averaging of its rounding, and the LSE bound is the single-score bound the window parity file derives.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))  # (the sibling parity files)
import test_parity as tj
import test_parity_adaln as ta
import test_parity_mlp as tm
import test_parity_streams as ts
import test_parity_varlen as tv
import test_parity_window as tw
from diffusion_transformer_joint_amd.inputs import (make_adaln_inputs, make_mlp_inputs, make_shape_inputs,
                                                    make_shape_stream_inputs, make_shape_varlen_inputs)

pytestmark = pytest.mark.gpu

HEAD_DIMS = (32, 64, 72, 128)


def say(msg):
    print(msg, flush=True)


def draw_mask(rng, B, L, few=True):
    """None, or per-sample lengths including the edges 0, L and past L (clamped by the library); with
    few=False no sample keeps fewer than half its keys (for checks without the single-score LSE bound)."""
    if rng.random() < 0.4:
        return None
    if few:
        return [int(rng.choice([0, 1, L, L + 3, rng.integers(0, L + 1)])) for _ in range(B)]
    return [int(rng.choice([0, L, L + 3, rng.integers((L + 1) // 2, L + 1)])) for _ in range(B)]


def lse_tol(inp):
    return max(tw.LSE_ABS, tw.single_score_lse_bound(inp))


@pytest.mark.parametrize("seed", range(100, 110))
def test_random_joint(seed):
    rng = np.random.default_rng(seed)
    B, L, H, D = int(rng.integers(1, 4)), int(rng.integers(1, 420)), int(rng.integers(1, 4)), int(rng.choice(HEAD_DIMS))
    vl = draw_mask(rng, B, L)
    say(f"case: random joint seed {seed}: B{B} L{L} H{H} D{D} valid_len={vl}")
    inp = make_shape_inputs(B, L, H, D, seed=seed, valid_len=vl)
    tw.check(tj.run_gpu(inp), tj.run_oracle(inp), tag=f"joint seed {seed}", lse_tol=lse_tol(inp))


@pytest.mark.parametrize("seed", range(200, 208))
def test_random_streams(seed):
    rng = np.random.default_rng(seed)
    B, H, D = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.choice(HEAD_DIMS))
    n_img = int(rng.choice([0, 1, 31, 64, rng.integers(2, 330)]))
    n_txt = int(rng.choice([0, 1, 77, rng.integers(2, 120)]))
    if n_img + n_txt == 0:
        n_txt = 5
    vl = draw_mask(rng, B, n_img + n_txt, few=False)
    say(f"case: random streams seed {seed}: B{B} n_img {n_img} n_txt {n_txt} H{H} D{D} valid_len={vl}")
    inp = make_shape_stream_inputs(B, n_img, n_txt, H, D, seed=seed, valid_len=vl)
    ts.check(ts.run_gpu(inp), ts.run_oracle(inp), tag=f"streams seed {seed}")


@pytest.mark.parametrize("seed", range(300, 308))
def test_random_varlen(seed):
    rng = np.random.default_rng(seed)
    H, D = int(rng.integers(1, 4)), int(rng.choice(HEAD_DIMS))
    lengths = [int(rng.choice([0, 64, rng.integers(16, 350)])) for _ in range(int(rng.integers(1, 6)))]
    if sum(lengths) == 0:
        lengths[0] = 17
    say(f"case: random varlen seed {seed}: lengths {lengths} H{H} D{D}")
    inp = make_shape_varlen_inputs(lengths, H, D, seed=seed)
    tv.check(tv.run_gpu(inp), tv.run_oracle(inp), inp["cu_seqlens"].tolist(), H, tag=f"varlen seed {seed}")


@pytest.mark.parametrize("seed", range(400, 408))
def test_random_window(seed):
    rng = np.random.default_rng(seed)
    B, L, H, D = int(rng.integers(1, 3)), int(rng.integers(2, 420)), int(rng.integers(1, 3)), int(rng.choice(HEAD_DIMS))
    side = lambda: int(rng.choice([-1, 1, 63, 64, rng.integers(1, 300)]))
    window = (side(), side())
    vl = draw_mask(rng, B, L)
    say(f"case: random window seed {seed}: B{B} L{L} H{H} D{D} window {window} valid_len={vl}")
    inp = make_shape_inputs(B, L, H, D, seed=seed, valid_len=vl)
    tw.check(tw.run_gpu(inp, window), tw.run_oracle(inp, window), tag=f"window seed {seed}", lse_tol=lse_tol(inp))


@pytest.mark.parametrize("seed", range(500, 505))
def test_random_adaln(seed):
    rng = np.random.default_rng(seed)
    B, C = int(rng.integers(1, 4)), 64 * int(rng.integers(1, 17))
    n_img, n_txt = int(rng.choice([0, 1, rng.integers(2, 300)])), int(rng.choice([0, 1, rng.integers(2, 90)]))
    if n_img + n_txt == 0:
        n_img = 9
    bias = bool(rng.random() < 0.7)
    say(f"case: random adaln seed {seed}: B{B} n_img {n_img} n_txt {n_txt} C{C} bias={bias}")
    inp = make_adaln_inputs(B, n_img, n_txt, C, seed=seed)
    got = ta.run_gpu(inp, bias=bias)
    for s, n in enumerate((n_img, n_txt)):
        if n:
            ta.check(got[s], ta.run_oracle(inp, s, bias=bias), f"adaln seed {seed} stream {s}")
        else:
            assert np.all(got[s]["dw"] == 0) and np.all(got[s]["dmod"] == 0)


@pytest.mark.parametrize("seed", range(600, 605))
def test_random_mlp(seed):
    rng = np.random.default_rng(seed)
    B, C, F = int(rng.integers(1, 4)), 64 * int(rng.integers(1, 9)), 64 * int(rng.integers(1, 17))
    n_img, n_txt = int(rng.choice([0, 1, rng.integers(2, 260)])), int(rng.choice([0, 1, rng.integers(2, 80)]))
    if n_img + n_txt == 0:
        n_txt = 11
    bias = bool(rng.random() < 0.7)
    say(f"case: random mlp seed {seed}: B{B} n_img {n_img} n_txt {n_txt} C{C} F{F} bias={bias}")
    inp = make_mlp_inputs(B, n_img, n_txt, C, F, seed=seed)
    got = tm.run_gpu(inp, bias=bias)
    for s, n in enumerate((n_img, n_txt)):
        if n:
            tm.check(got[s], tm.run_oracle(inp, s, bias=bias), inp, s, f"mlp seed {seed} stream {s}")
        else:
            for k in ("dmod", "dwfc", "dw12", "dw2"):
                assert np.all(got[s][k] == 0), k
