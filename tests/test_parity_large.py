"""GPU parity at sizes where a 32-bit element offset would overflow: the attention on a batch of
4096 x 1024 tokens x 16 heads x 64 (2^32 elements per tensor, 8.6 GB), the adaLN projection with
T * 3C just under 2^31, and the MLP block with T * 2F just under 2^31.

The inputs are drawn on the GPU from a seeded torch generator (drawing tens of GB on the host would
take minutes); only the sampled rows or (batch, head) pairs are copied back for the oracle, which
computes them exactly because pairs (attention) and token rows (per-row outputs of the projections)
are independent. Sums over all tokens are checked through exact column sums and the Euler identity
of the linear parameters, as in the full-workload tests. Tolerances are those of each family."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))  # (the sibling parity files)
import test_parity as tj
import test_parity_adaln as ta
import test_parity_mlp as tm
from diffusion_transformer_joint_amd import adaln, mlp, ops
from diffusion_transformer_joint_amd.inputs import default_scale
from oracle import adaln_qkv_fwd_bwd, attention_fwd_bwd, mlp_fwd_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def release_memory():
    """These tests hold tens of GB; hand the cached blocks back so later tests start from a clean pool."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(msg):
    print(msg, flush=True)


def gen(seed):
    return torch.Generator(device="cuda:0").manual_seed(seed)


def f64(t):
    return t.double().cpu().numpy()


def test_attention_batch_past_2pow32_elements():
    B, L, H, D = 4096, 1024, 16, 64
    say(f"case: large joint attention B{B} L{L} H{H} D{D} (2^32 elements per tensor), seed 11")
    dev = torch.device("cuda:0")
    g = gen(11)
    q, k, v, dout = (torch.randn(B, L, H, D, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(4))
    gains = (1.0 + 0.1 * torch.randn(2, D, device=dev, generator=g)).float()
    scale, eps = default_scale(D), 1e-6
    out, lse, fws = ops.forward(q, k, v, gains, None, scale, eps, return_workspace=True)
    dq, dk, dv, _ = ops.backward(q, k, v, gains, out, lse, dout, None, scale, eps, fwd_workspace=fws)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (2047, 9), (B - 1, H - 1)):
        sl = lambda t: f64(t[b:b + 1, :, h:h + 1, :])
        ref = attention_fwd_bwd(sl(q), sl(k), sl(v), f64(gains), sl(dout), None, scale, eps)
        got = dict(out=sl(out), lse=f64(lse[b:b + 1, h:h + 1]), dq=sl(dq), dk=sl(dk), dv=sl(dv),
                   dgains=ref["dgains"])  # (dgains sums over every pair: not compared here)
        tj.check(got, ref, tag=f"large joint pair b{b} h{h}")


def test_adaln_rows_near_the_limit():
    B, n_img, n_txt, C = 1, 233000, 10, 3072
    say(f"case: large adaln B{B} n_img {n_img} n_txt {n_txt} C{C} (T * 3C just under 2^31), seed 12")
    dev = torch.device("cuda:0")
    g = gen(12)
    ns = (n_img, n_txt)
    x = tuple(torch.randn(B, n, C, device=dev, dtype=torch.bfloat16, generator=g) for n in ns)
    mod = tuple(0.2 * torch.randn(B, 2, C, device=dev, generator=g) for _ in ns)
    w = tuple(((2 * torch.rand(3 * C, C, device=dev, generator=g) - 1) / C ** 0.5).bfloat16() for _ in ns)
    bias = tuple((2 * torch.rand(3 * C, device=dev, generator=g) - 1) / C ** 0.5 for _ in ns)
    dy = [tuple(torch.randn(B, n, C, device=dev, dtype=torch.bfloat16, generator=g) for n in ns) for _ in range(3)]
    q, k, v, ws = adaln.adaln_qkv_forward(x, mod, w, bias, 1e-6)
    dx, dmod, dw, db = adaln.adaln_qkv_backward(x, mod, w, dy[0], dy[1], dy[2], ws)
    torch.cuda.synchronize()
    s = 0
    rows = [0, 1, 117001, n_img - 1]
    idx = torch.tensor(rows, device=dev)
    take = lambda t: f64(t[s].index_select(1, idx))
    ref = adaln_qkv_fwd_bwd(take(x), f64(mod[s]), f64(w[s]), f64(bias[s]), 1, 1e-6,
                            *(take(t).reshape(B, len(rows), 1, C) for t in dy))
    got = dict(q=take(q), k=take(k), v=take(v), dx=take(dx))
    ta.check(got, ref, f"large adaln rows {rows}", keys=("q", "k", "v", "dx"))
    # sums over all tokens: the bias gradient is the column sum of [dq | dk | dv]; the weight and bias
    # gradients together satisfy <dW, W> + <db, b> = sum(dY * Y)
    dycat = torch.cat([t[s].reshape(-1, C) for t in dy], dim=1).double()
    colsum = dycat.sum(dim=0)
    assert tj.rel_l2(f64(db[s]), colsum.cpu().numpy()) <= 1e-5
    ycat = torch.cat([t[s].reshape(-1, C) for t in (q, k, v)], dim=1).double()
    lhs = float((dw[s].double() * w[s].double()).sum() + (db[s].double() * bias[s].double()).sum())
    rhs = float((dycat * ycat).sum())
    say(f"large adaln: <dW,W>+<db,b> {lhs:.6e} vs sum(dY*Y) {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-2 * float(dycat.norm()) * float(ycat.norm())


def test_mlp_rows_near_the_limit():
    B, n_img, n_txt, C, F = 1, 131000, 60, 3072, 8192
    say(f"case: large mlp B{B} n_img {n_img} n_txt {n_txt} C{C} F{F} (T * 2F just under 2^31), seed 13")
    dev = torch.device("cuda:0")
    g = gen(13)
    ns = (n_img, n_txt)
    u = lambda shape, fan: (2 * torch.rand(*shape, device=dev, generator=g) - 1) / fan ** 0.5
    o = tuple(torch.randn(B, n, C, device=dev, dtype=torch.bfloat16, generator=g) for n in ns)
    x = tuple(torch.randn(B, n, C, device=dev, dtype=torch.bfloat16, generator=g) for n in ns)
    mod = tuple(0.2 * torch.randn(B, 2, C, device=dev, generator=g) for _ in ns)
    wfc = tuple(u((C, C), C).bfloat16() for _ in ns)
    bfc = tuple(u((C,), C) for _ in ns)
    w12 = tuple(u((2 * F, C), C).bfloat16() for _ in ns)
    b12 = tuple(u((2 * F,), C) for _ in ns)
    w2 = tuple(u((C, F), F).bfloat16() for _ in ns)
    b2 = tuple(u((C,), F) for _ in ns)
    dout = tuple(torch.randn(B, n, C, device=dev, dtype=torch.bfloat16, generator=g) for n in ns)
    eps = 1e-6
    out, ws = mlp.mlp_forward(o, x, mod, wfc, w12, w2, bfc, b12, b2, eps)
    gr = mlp.mlp_backward(o, mod, wfc, w12, w2, dout, ws)
    torch.cuda.synchronize()
    del ws
    s = 0
    rows = [0, 65537, n_img - 1]
    idx = torch.tensor(rows, device=dev)
    take = lambda t: f64(t[s].index_select(1, idx))
    ref = mlp_fwd_bwd(take(o), take(x), f64(mod[s]), f64(wfc[s]), f64(bfc[s]), f64(w12[s]), f64(b12[s]), f64(w2[s]),
                      f64(b2[s]), eps, take(dout))
    got_out, got_do, ref_out, ref_do = take(out), take(gr["do"]), ref["out"], ref["do"]
    errs = dict(out=tm.rel_l2(got_out, ref_out), out_abs=float(np.max(np.abs(got_out - ref_out))),
                do=tm.rel_l2(got_do, ref_do))
    say(f"large mlp rows {rows}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["out"] <= tm.OUT_REL and errs["out_abs"] <= tm.OUT_ABS and errs["do"] <= tm.DO_REL, errs
    # db2 is the column sum of dout; <dW2, W2> + <db2, b2> = sum(dout * y) with y the block's own part
    dflat = dout[s].reshape(-1, C).double()
    assert tm.rel_l2(f64(gr["db2"][s]), dflat.sum(dim=0).cpu().numpy()) <= 1e-5
    zero = tuple(torch.zeros_like(t) for t in x)
    y, _ = mlp.mlp_forward(o, zero, mod, wfc, w12, w2, bfc, b12, b2, eps)
    torch.cuda.synchronize()
    yflat = y[s].reshape(-1, C).double()
    lhs = float((gr["dw2"][s].double() * w2[s].double()).sum() + (gr["db2"][s].double() * b2[s].double()).sum())
    rhs = float((dflat * yflat).sum())
    say(f"large mlp: <dW2,W2>+<db2,b2> {lhs:.6e} vs sum(dout*y) {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-2 * float(dflat.norm()) * float(yflat.norm())
