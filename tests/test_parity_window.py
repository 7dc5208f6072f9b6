"""GPU parity of the local-window entry points (query i sees keys i - left .. i + right, besides the
key padding) against the fp64 oracle's window option on the same seeded inputs, with the joint form's
tolerances: out relative L2 <= 5e-3 and max abs <= 2e-2, LSE max abs <= 1e-2 with -inf exactly where
a row's window holds no valid key, relative L2 <= 1e-2 for dq, dk, dv and dgains."""
import json
import os

import numpy as np
import pytest
import torch

from diffusion_transformer_joint_amd import ops
from diffusion_transformer_joint_amd.inputs import WORKLOADS, make_inputs, make_shape_inputs
from oracle import attention_fwd_bwd

pytestmark = pytest.mark.gpu

FWD_REL, FWD_ABS, BWD_REL, LSE_ABS = 5e-3, 2e-2, 1e-2, 1e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(msg):
    print(msg, flush=True)


def run_gpu(inp, window):
    dev = torch.device("cuda:0")
    d = {k: inp[k].to(dev).contiguous() for k in ("q", "k", "v", "gains", "dout")}
    vl = None if inp["valid_len"] is None else inp["valid_len"].to(dev)
    out, lse, fws = ops.forward(d["q"], d["k"], d["v"], d["gains"], vl, inp["scale"], inp["eps"], return_workspace=True,
                                window=window)
    dq, dk, dv, dg = ops.backward(d["q"], d["k"], d["v"], d["gains"], out, lse, d["dout"], vl, inp["scale"],
                                  inp["eps"], fwd_workspace=fws, window=window)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return dict(out=f(out), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv), dgains=f(dg))


def run_oracle(inp, window, pairs=None):
    f = lambda t: t.to(torch.float64).numpy()
    vl = None if inp["valid_len"] is None else inp["valid_len"].tolist()
    return attention_fwd_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["gains"].double().numpy(), f(inp["dout"]), vl,
                             inp["scale"], inp["eps"], pairs=pairs, window=window)


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


def check(got, ref, pairs=None, dgains_ref=None, tag="", lse_tol=LSE_ABS):
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
    assert errs["lse_abs"] <= lse_tol, (tag, errs)
    for key in ("dq", "dk", "dv", "dgains"):
        assert errs[key] <= BWD_REL, (tag, key, errs)
    return errs


SHAPES = [
    # B, L, H, D, valid_len, window
    (2, 300, 2, 64, [300, 200], (64, 64)),
    (1, 513, 2, 128, None, (-1, 0)),        # causal
    (2, 200, 2, 72, [200, 150], (0, 0)),    # zero width
    (1, 257, 3, 32, [150], (100, 30)),      # rows past the keys with nothing in their window
    (2, 1101, 2, 64, None, (300, 40)),
    (1, 130, 2, 64, [100], (1000, 1000)),   # wider than the sequence
]


def single_score_lse_bound(inp):
    """A row with one key in its window has LSE = that one score, with no averaging over keys: its
    error is the score's own bf16 operand rounding, |dS| <= scale * 2^-8 * |Qn_i| |Kn_i| (relative 2^-9 on
    each operand element)."""
    q, k, g = (inp[n].double().numpy() for n in ("q", "k", "gains"))
    nq = np.linalg.norm(q / np.sqrt(np.mean(q ** 2, axis=-1, keepdims=True) + inp["eps"]) * g[0], axis=-1)
    nk = np.linalg.norm(k / np.sqrt(np.mean(k ** 2, axis=-1, keepdims=True) + inp["eps"]) * g[1], axis=-1)
    return abs(inp["scale"]) * 2.0 ** -8 * float(np.max(nq * nk))


@pytest.mark.parametrize("B,L,H,D,vl,window", SHAPES)
def test_window_shapes(B, L, H, D, vl, window):
    say(f"case: window {window} B{B} L{L} H{H} D{D} valid_len={vl}, seed 1")
    inp = make_shape_inputs(B, L, H, D, seed=1, valid_len=vl)
    got = run_gpu(inp, window)
    tol = max(LSE_ABS, single_score_lse_bound(inp)) if window == (0, 0) else LSE_ABS
    check(got, run_oracle(inp, window), tag=f"window {window} B{B}L{L}D{D}", lse_tol=tol)
    if vl is not None:   # padded keys still get exact zeros
        for b, n in enumerate(vl):
            assert np.all(got["dk"][b, n:] == 0) and np.all(got["dv"][b, n:] == 0)


def test_window_rows_without_keys_are_zero():
    """valid_len 40 and window (5, 5): row i sees keys i - 5 .. i + 5 below 40, so rows 45 .. 99 see none:
    out = 0 and lse = -inf exactly; rows 0 .. 44 see at least one."""
    say("case: window (5, 5) B1 L100 H2 D64 valid_len [40]")
    inp = make_shape_inputs(1, 100, 2, 64, seed=2, valid_len=[40])
    got = run_gpu(inp, (5, 5))
    assert np.all(got["out"][0, 45:] == 0) and np.all(np.isneginf(got["lse"][0, :, 45:]))
    assert np.all(np.isfinite(got["lse"][0, :, :45]))
    check(got, run_oracle(inp, (5, 5)), tag="window empty rows")


def test_window_full_workload():
    """The headline workload with a 256-token window each way: sampled pairs, and the gain gradients
    against the stored oracle values."""
    w = WORKLOADS["mmdit512"]
    say(f"case: window (256, 256) full workload mmdit512 B{w.B} L{w.L} H{w.H} D{w.D}, seed 0")
    inp = make_inputs("mmdit512", seed=0)
    got = run_gpu(inp, (256, 256))
    pairs = sorted({(0, 0), (w.B // 2, w.H // 2), (w.B - 1, w.H - 1)})
    with open(os.path.join(GOLDEN, "dgains_window_mmdit512.json")) as f:
        gold = json.load(f)
    assert gold["window"] == [256, 256]
    check(got, run_oracle(inp, (256, 256), pairs=pairs), pairs=pairs, dgains_ref=np.array(gold["dgains"]),
          tag="window mmdit512")


def test_window_deterministic_and_autograd():
    say("case: window determinism and autograd B1 L300 H2 D64 window (50, 20)")
    inp = make_shape_inputs(1, 300, 2, 64, seed=3, valid_len=[270])
    dev = torch.device("cuda:0")
    d = {k: inp[k].to(dev).contiguous() for k in ("q", "k", "v", "gains", "dout")}
    vl = inp["valid_len"].to(dev)
    q, k, v, g = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "gains"))
    o = ops.joint_attention(q, k, v, g, vl, inp["scale"], inp["eps"], window=(50, 20))
    o.backward(d["dout"])
    out, lse = ops.forward(d["q"], d["k"], d["v"], d["gains"], vl, inp["scale"], inp["eps"], window=(50, 20))
    r1 = [t.clone() for t in ops.backward(d["q"], d["k"], d["v"], d["gains"], out, lse, d["dout"], vl, inp["scale"],
                                          inp["eps"], window=(50, 20))]
    r2 = ops.backward(d["q"], d["k"], d["v"], d["gains"], out, lse, d["dout"], vl, inp["scale"], inp["eps"],
                      window=(50, 20))
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), out)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    for a, b in zip((q.grad, k.grad, v.grad, g.grad), r1):
        assert torch.equal(a, b)
