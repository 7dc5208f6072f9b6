"""GPU parity of every compiled head dim (each multiple of 8 from 32 to 128) in the four attention
forms, against the fp64 oracle. The head dim sets the padded contraction and output widths of the
kernels (multiples of 16 and 32), the LDS layout and the staging layout, so each value is its own
instantiation; the shapes span several 64-key and 128-row tiles with ragged tails, a key mask that
cuts inside a tile, and a text stream shorter than a tile. Tolerances and comparisons are those of
each form's own parity file (imported from it)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))  # (the sibling parity files)
import test_parity as tj
import test_parity_streams as ts
import test_parity_varlen as tv
import test_parity_window as tw
from diffusion_transformer_joint_amd.inputs import (make_shape_inputs, make_shape_stream_inputs,
                                                    make_shape_varlen_inputs)

pytestmark = pytest.mark.gpu

HEAD_DIMS = tuple(range(32, 129, 8))


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_head_dim_joint(D):
    say(f"case: joint B2 L300 H2 D{D} valid_len [300, 171], seed {700 + D}")
    inp = make_shape_inputs(2, 300, 2, D, seed=700 + D, valid_len=[300, 171])
    tj.check(tj.run_gpu(inp), tj.run_oracle(inp), tag=f"joint D{D}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_head_dim_streams(D):
    say(f"case: two-stream B2 n_img 200 n_txt 45 H2 D{D}, seed {800 + D}")
    inp = make_shape_stream_inputs(2, 200, 45, 2, D, seed=800 + D)
    ts.check(ts.run_gpu(inp), ts.run_oracle(inp), tag=f"streams D{D}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_head_dim_varlen(D):
    lengths = [190, 0, 77, 261]
    say(f"case: varlen lengths {lengths} H2 D{D}, seed {900 + D}")
    inp = make_shape_varlen_inputs(lengths, 2, D, seed=900 + D)
    tv.check(tv.run_gpu(inp), tv.run_oracle(inp), inp["cu_seqlens"].tolist(), 2, tag=f"varlen D{D}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_head_dim_window(D):
    window = (70, 33)
    say(f"case: window {window} B1 L333 H2 D{D}, seed {1000 + D}")
    inp = make_shape_inputs(1, 333, 2, D, seed=1000 + D)
    tw.check(tw.run_gpu(inp, window), tw.run_oracle(inp, window), tag=f"window D{D}")
