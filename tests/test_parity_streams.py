"""GPU parity of the two-stream entry points (image and text tokens in their own tensors, a QK-norm
gain pair per stream) against the fp64 two-stream oracle on the same seeded inputs. Tolerances are
those of the joint form: forward out relative L2 <= 5e-3 and max abs <= 2e-2, LSE max abs <= 1e-2,
backward relative L2 <= 1e-2 for dq, dk, dv (both stream parts together) and dgains.

The shapes put the stream boundary inside a 64-row tile (so the boundary tile is loaded from both
streams' tensors), on a tile edge, past the last valid key, and at either end (one stream empty)."""
import json
import os

import numpy as np
import pytest
import torch

from diffusion_transformer_joint_amd import ops
from diffusion_transformer_joint_amd.inputs import WORKLOADS, make_shape_stream_inputs, make_stream_inputs
from oracle import streams_fwd_bwd

pytestmark = pytest.mark.gpu

FWD_REL, FWD_ABS, BWD_REL, LSE_ABS = 5e-3, 2e-2, 1e-2, 1e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(msg):
    print(msg, flush=True)


def to_dev(inp):
    dev = torch.device("cuda:0")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in ("q", "k", "v", "dout")}
    d["gains"] = inp["gains"].to(dev)
    d["valid_len"] = None if inp["valid_len"] is None else inp["valid_len"].to(dev)
    return d


def run_gpu(inp):
    d = to_dev(inp)
    out, lse, fws = ops.forward_streams(d["q"], d["k"], d["v"], d["gains"], d["valid_len"], inp["scale"],
                                        inp["eps"], return_workspace=True)
    dq, dk, dv, dg = ops.backward_streams(d["q"], d["k"], d["v"], d["gains"], out, lse, d["dout"], d["valid_len"],
                                          inp["scale"], inp["eps"], fwd_workspace=fws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    cat = lambda p: np.concatenate([f(p[0]), f(p[1])], axis=1)
    return dict(out=cat(out), lse=f(lse), dq=cat(dq), dk=cat(dk), dv=cat(dv), dgains=f(dg))


def run_oracle(inp, pairs=None):
    f = lambda t: t.to(torch.float64).numpy()
    pair = lambda key: (f(inp[key][0]), f(inp[key][1]))
    vl = None if inp["valid_len"] is None else inp["valid_len"].tolist()
    r = streams_fwd_bwd(pair("q"), pair("k"), pair("v"), inp["gains"].double().numpy(), pair("dout"), vl,
                        inp["scale"], inp["eps"], pairs=pairs)
    cat = lambda p: np.concatenate(p, axis=1)
    return dict(out=cat(r["out"]), lse=r["lse"], dq=cat(r["dq"]), dk=cat(r["dk"]), dv=cat(r["dv"]),
                dgains=r["dgains"])


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def select(t, pairs, key):
    if pairs is None:
        return t.ravel()
    if key == "lse":
        return np.concatenate([t[b, h].ravel() for b, h in pairs])
    return np.concatenate([t[b, :, h].ravel() for b, h in pairs])


def check(got, ref, pairs=None, dgains_ref=None, tag=""):
    errs = {}
    o, ro = select(got["out"], pairs, "out"), select(ref["out"], pairs, "out")
    errs["out_rel"], errs["out_abs"] = rel_l2(o, ro), float(np.max(np.abs(o - ro)))
    l, rl = select(got["lse"], pairs, "lse"), select(ref["lse"], pairs, "lse")
    assert np.array_equal(np.isneginf(l), np.isneginf(rl)), f"{tag}: -inf rows differ"
    fin = np.isfinite(rl)
    errs["lse_abs"] = float(np.max(np.abs(l[fin] - rl[fin]))) if fin.any() else 0.0
    for key in ("dq", "dk", "dv"):
        errs[key] = rel_l2(select(got[key], pairs, key), select(ref[key], pairs, key))
    errs["dgains"] = rel_l2(got["dgains"], ref["dgains"] if dgains_ref is None else dgains_ref)
    say(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["out_rel"] <= FWD_REL and errs["out_abs"] <= FWD_ABS, (tag, errs)
    assert errs["lse_abs"] <= LSE_ABS, (tag, errs)
    for key in ("dq", "dk", "dv", "dgains"):
        assert errs[key] <= BWD_REL, (tag, key, errs)
    return errs


SHAPES = [
    # B, n_img, n_txt, H, D, valid_len
    (2, 100, 37, 2, 64, None),            # boundary inside a tile (row 100 of tile 64..127)
    (2, 130, 70, 3, 128, [200, 150]),     # padded text keys
    (1, 64, 77, 2, 72, [100]),            # boundary on a tile edge
    (2, 16, 8, 2, 32, None),              # the tiny patch-grid shape
    (2, 100, 37, 2, 64, [90, 137]),       # sequence 0: no valid text key
    (1, 300, 0, 2, 64, [250]),            # no text stream
    (2, 0, 77, 2, 128, None),             # no image stream
    (1, 1, 200, 1, 64, None),             # one image token
]


@pytest.mark.parametrize("B,n_img,n_txt,H,D,vl", SHAPES)
def test_streams_shapes(B, n_img, n_txt, H, D, vl):
    say(f"case: two-stream B{B} img{n_img} txt{n_txt} H{H} D{D} valid_len={vl}, seed 1")
    inp = make_shape_stream_inputs(B, n_img, n_txt, H, D, seed=1, valid_len=vl, gain_std=0.3)
    check(run_gpu(inp), run_oracle(inp), tag=f"streams B{B}I{n_img}T{n_txt}H{H}D{D}")


def test_streams_tiny_workload():
    say("case: two-stream tiny workload (16 image + 8 text tokens), seed 0")
    inp = make_stream_inputs("tiny", seed=0)
    check(run_gpu(inp), run_oracle(inp), tag="streams tiny")


def test_streams_full_mmdit512():
    """The headline workload in two-stream form: per-token outputs on sampled (batch, head) pairs, the
    gain gradients (a sum over all pairs) against the stored oracle values."""
    w = WORKLOADS["mmdit512"]
    say(f"case: two-stream full workload mmdit512 B{w.B} img{w.n_img} txt{w.n_txt} H{w.H} D{w.D}, seed 0")
    inp = make_stream_inputs("mmdit512", seed=0)
    got = run_gpu(inp)
    pairs = sorted({(0, 0), (w.B // 2, w.H // 2), (w.B - 1, w.H - 1)})
    ref = run_oracle(inp, pairs=pairs)
    with open(os.path.join(GOLDEN, "dgains_streams_mmdit512.json")) as f:
        gold = json.load(f)
    assert gold["B"] == w.B and gold["n_img"] == w.n_img and gold["n_txt"] == w.n_txt
    check(got, ref, pairs=pairs, dgains_ref=np.array(gold["dgains"]), tag="streams mmdit512")


def test_streams_match_joint_with_shared_gains():
    """With both streams given the same gains, the two-stream call computes the joint attention of the
    concatenated tensors: both are held to the oracle, and to each other at twice the tolerance."""
    say("case: two-stream vs joint, shared gains, B2 img100 txt37 H2 D64")
    inp = make_shape_stream_inputs(2, 100, 37, 2, 64, seed=2, valid_len=[137, 120])
    inp["gains"][1] = inp["gains"][0]
    s = run_gpu(inp)
    d = to_dev(inp)
    cat = lambda p: torch.cat(p, dim=1).contiguous()
    out, lse = ops.forward(cat(d["q"]), cat(d["k"]), cat(d["v"]), d["gains"][0].contiguous(), d["valid_len"],
                           inp["scale"], inp["eps"])
    dq, dk, dv, dg = ops.backward(cat(d["q"]), cat(d["k"]), cat(d["v"]), d["gains"][0].contiguous(), out, lse,
                                  cat(d["dout"]), d["valid_len"], inp["scale"], inp["eps"])
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    assert rel_l2(s["out"], f(out)) <= 2 * FWD_REL
    for key, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert rel_l2(s[key], f(t)) <= 2 * BWD_REL, key
    assert rel_l2(s["dgains"][0] + s["dgains"][1], f(dg)) <= 2 * BWD_REL
    check(s, run_oracle(inp), tag="streams shared-gains")


def test_streams_backward_is_deterministic_and_autograd():
    say("case: two-stream determinism and autograd B2 img90 txt50 H2 D64")
    inp = make_shape_stream_inputs(2, 90, 50, 2, 64, seed=3, valid_len=[140, 101])
    d = to_dev(inp)
    leaves = [t.clone().requires_grad_(True) for t in (*d["q"], *d["k"], *d["v"], d["gains"])]
    qi, qt, ki, kt, vi, vt, g = leaves
    o_img, o_txt = ops.joint_attention_streams((qi, qt), (ki, kt), (vi, vt), g, d["valid_len"], inp["scale"],
                                               inp["eps"])
    torch.autograd.backward([o_img, o_txt], [d["dout"][0], d["dout"][1]])
    out, lse = ops.forward_streams(d["q"], d["k"], d["v"], d["gains"], d["valid_len"], inp["scale"], inp["eps"])
    r1 = ops.backward_streams(d["q"], d["k"], d["v"], d["gains"], out, lse, d["dout"], d["valid_len"], inp["scale"],
                              inp["eps"])
    r2 = ops.backward_streams(d["q"], d["k"], d["v"], d["gains"], out, lse, d["dout"], d["valid_len"], inp["scale"],
                              inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(o_img.detach(), out[0]) and torch.equal(o_txt.detach(), out[1])
    for a, b in zip(r1[:3], r2[:3]):
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(r1[3], r2[3])
    grads = [qi.grad, qt.grad, ki.grad, kt.grad, vi.grad, vt.grad]
    want = [r1[0][0], r1[0][1], r1[1][0], r1[1][1], r1[2][0], r1[2][1]]
    for a, b in zip(grads, want):
        assert torch.equal(a, b)
    assert torch.equal(g.grad, r1[3])
