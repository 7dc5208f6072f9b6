"""GPU parity of the packed variable-length entry points (sequences back to back in [total, H, D]
tensors, cu_seqlens offsets) against the fp64 variable-length oracle on the same seeded inputs, with
the joint form's tolerances: out relative L2 <= 5e-3 and max abs <= 2e-2, LSE max abs <= 1e-2,
relative L2 <= 1e-2 for dq, dk, dv and dgains."""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

from diffusion_transformer_joint_amd import _lib, ops
from diffusion_transformer_joint_amd.inputs import VARLEN_WORKLOADS, make_shape_varlen_inputs, make_varlen_inputs
from oracle import varlen_fwd_bwd

pytestmark = pytest.mark.gpu

FWD_REL, FWD_ABS, BWD_REL, LSE_ABS = 5e-3, 2e-2, 1e-2, 1e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(msg):
    print(msg, flush=True)


def to_dev(inp):
    dev = torch.device("cuda:0")
    d = {k: inp[k].to(dev).contiguous() for k in ("q", "k", "v", "dout", "gains", "cu_seqlens")}
    return d


def run_gpu(inp, max_seqlen=None):
    d = to_dev(inp)
    ms = inp["max_seqlen"] if max_seqlen is None else max_seqlen
    out, lse, fws = ops.forward_varlen(d["q"], d["k"], d["v"], d["gains"], d["cu_seqlens"], ms, inp["scale"],
                                       inp["eps"], return_workspace=True)
    dq, dk, dv, dg = ops.backward_varlen(d["q"], d["k"], d["v"], d["gains"], d["cu_seqlens"], ms, out, lse, d["dout"],
                                         inp["scale"], inp["eps"], fwd_workspace=fws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return dict(out=f(out), lse=f(lse), dq=f(dq), dk=f(dk), dv=f(dv), dgains=f(dg))


def run_oracle(inp, seqs=None):
    f = lambda t: t.to(torch.float64).numpy()
    return varlen_fwd_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["gains"].double().numpy(), f(inp["dout"]),
                          inp["cu_seqlens"].tolist(), inp["scale"], inp["eps"], seqs=seqs)


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def check(got, ref, cu, H, seqs=None, dgains_ref=None, tag=""):
    B = len(cu) - 1
    seqs = [b for b in range(B) if cu[b + 1] > cu[b]] if seqs is None else seqs
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in seqs]) if seqs else np.zeros(0, dtype=int)
    errs = {}
    o, ro = got["out"][rows].ravel(), ref["out"][rows].ravel()
    errs["out_rel"], errs["out_abs"] = rel_l2(o, ro), float(np.max(np.abs(o - ro))) if o.size else 0.0
    lse_err = 0.0
    for b in seqs:
        L = cu[b + 1] - cu[b]
        g = got["lse"][cu[b] * H:cu[b + 1] * H].reshape(H, L)
        lse_err = max(lse_err, float(np.max(np.abs(g - ref["lse"][b]))))
    errs["lse_abs"] = lse_err
    for key in ("dq", "dk", "dv"):
        errs[key] = rel_l2(got[key][rows].ravel(), ref[key][rows].ravel())
    errs["dgains"] = rel_l2(got["dgains"], ref["dgains"] if dgains_ref is None else dgains_ref)
    say(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["out_rel"] <= FWD_REL and errs["out_abs"] <= FWD_ABS, (tag, errs)
    assert errs["lse_abs"] <= LSE_ABS, (tag, errs)
    for key in ("dq", "dk", "dv", "dgains"):
        assert errs[key] <= BWD_REL, (tag, key, errs)


SHAPES = [
    # lengths, H, D
    ([37, 200, 1, 129], 2, 64),
    ([0, 70, 0, 257], 2, 128),     # empty sequences
    ([300, 150], 3, 72),
    ([64, 64, 65], 2, 32),
    ([513], 1, 64),
]


@pytest.mark.parametrize("lengths,H,D", SHAPES)
def test_varlen_shapes(lengths, H, D):
    say(f"case: varlen lengths {lengths} H{H} D{D}, seed 1")
    inp = make_shape_varlen_inputs(lengths, H, D, seed=1, gain_std=0.3)
    check(run_gpu(inp), run_oracle(inp), inp["cu_seqlens"].tolist(), H, tag=f"varlen {lengths} D{D}")


def test_varlen_loose_max_seqlen():
    """max_seqlen above the longest sequence: the extra row blocks of every sequence do nothing."""
    say("case: varlen lengths [90, 33] H2 D64, max_seqlen 400")
    inp = make_shape_varlen_inputs([90, 33], 2, 64, seed=2)
    check(run_gpu(inp, max_seqlen=400), run_oracle(inp), inp["cu_seqlens"].tolist(), 2, tag="varlen loose max")


def test_varlen_offsets_are_clamped():
    """cu_seqlens = [0, 100, 160] with max_seqlen 80: the first sequence is cut to its first 80 rows
    (rows 80..99 are not written), the second keeps its 60; results are those of [0, 80] and [100, 160]."""
    say("case: varlen clamping cu [0, 100, 160], max_seqlen 80, H2 D64")
    inp = make_shape_varlen_inputs([100, 60], 2, 64, seed=3)
    d = to_dev(inp)
    total, H, D = 160, 2, 64
    lib = _lib.load()
    out = torch.full((total, H, D), 7.0, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((total * H,), 7.0, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(int(lib.jattn_varlen_fwd_workspace_bytes(2, 80, total, H, D)), dtype=torch.uint8,
                     device="cuda:0")
    st = lib.jattn_fwd_varlen(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["gains"].data_ptr(),
                              d["cu_seqlens"].data_ptr(), 2, 80, total, H, D, ctypes.c_float(inp["scale"]),
                              ctypes.c_float(inp["eps"]), out.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(),
                              None, 0, torch.cuda.current_stream().cuda_stream)
    _lib.check("jattn_fwd_varlen", st)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(got[80:100] == 7.0)
    f = lambda t: t.to(torch.float64).numpy()
    for r0, r1 in ((0, 80), (100, 160)):
        ref = varlen_fwd_bwd(f(inp["q"][r0:r1]), f(inp["k"][r0:r1]), f(inp["v"][r0:r1]), inp["gains"].double().numpy(),
                             f(inp["dout"][r0:r1]), [0, r1 - r0], inp["scale"], inp["eps"])
        assert rel_l2(got[r0:r1].ravel(), ref["out"].ravel()) <= FWD_REL
        g = lse.cpu().numpy()[r0 * H:r0 * H + H * (r1 - r0)].reshape(H, r1 - r0)
        assert np.max(np.abs(g - ref["lse"][0])) <= LSE_ABS


@pytest.mark.parametrize("name", ["varlen_multires", "varlen_ragged"])
def test_varlen_full_workload(name):
    w = VARLEN_WORKLOADS[name]
    say(f"case: full varlen workload {name} B{w.B} H{w.H} D{w.D}, seed 0")
    inp = make_varlen_inputs(name, seed=0)
    got = run_gpu(inp)
    B = w.B
    seqs = sorted({0, B // 2, B - 1})
    ref = run_oracle(inp, seqs=seqs)
    with open(os.path.join(GOLDEN, f"dgains_{name}.json")) as fh:
        gold = json.load(fh)
    assert gold["lengths"] == inp["lengths"]
    check(got, ref, inp["cu_seqlens"].tolist(), w.H, seqs=seqs, dgains_ref=np.array(gold["dgains"]), tag=name)


def test_varlen_matches_padded_joint_path():
    """The same sequences padded to the longest, keys masked by valid_len and dout zero on the padded
    rows, through the joint entry points: the real rows agree with the packed results to twice the
    parity tolerance."""
    say("case: varlen vs padded joint path, lengths [120, 33, 200] H2 D64")
    lengths = [120, 33, 200]
    inp = make_shape_varlen_inputs(lengths, 2, 64, seed=4)
    v = run_gpu(inp)
    cu = inp["cu_seqlens"].tolist()
    Lm, H, D = max(lengths), 2, 64
    pad = lambda t: torch.stack([torch.cat([t[cu[b]:cu[b + 1]], torch.zeros(Lm - n, H, D, dtype=t.dtype)])
                                 for b, n in enumerate(lengths)]).cuda()
    vl = torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    g = inp["gains"].cuda()
    out, lse = ops.forward(pad(inp["q"]), pad(inp["k"]), pad(inp["v"]), g, vl, inp["scale"], inp["eps"])
    dq, dk, dv, dg = ops.backward(pad(inp["q"]), pad(inp["k"]), pad(inp["v"]), g, out, lse, pad(inp["dout"]), vl,
                                  inp["scale"], inp["eps"])
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    unpad = lambda t: np.concatenate([f(t)[b, :n] for b, n in enumerate(lengths)])
    for key, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert rel_l2(v[key], unpad(t)) <= 2 * (FWD_REL if key == "out" else BWD_REL), key
    assert rel_l2(v["dgains"], f(dg)) <= 2 * BWD_REL


def test_varlen_deterministic_and_autograd():
    say("case: varlen determinism and autograd, lengths [150, 77, 201] H2 D64")
    inp = make_shape_varlen_inputs([150, 77, 201], 2, 64, seed=5)
    d = to_dev(inp)
    ms = inp["max_seqlen"]
    q, k, v, g = (d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "gains"))
    o = ops.joint_attention_varlen(q, k, v, g, d["cu_seqlens"], ms, inp["scale"], inp["eps"])
    o.backward(d["dout"])
    out, lse = ops.forward_varlen(d["q"], d["k"], d["v"], d["gains"], d["cu_seqlens"], ms, inp["scale"], inp["eps"])
    r1 = ops.backward_varlen(d["q"], d["k"], d["v"], d["gains"], d["cu_seqlens"], ms, out, lse, d["dout"],
                             inp["scale"], inp["eps"])
    r1 = [t.clone() for t in r1]
    r2 = ops.backward_varlen(d["q"], d["k"], d["v"], d["gains"], d["cu_seqlens"], ms, out, lse, d["dout"],
                             inp["scale"], inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), out)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    for a, b in zip((q.grad, k.grad, v.grad, g.grad), r1):
        assert torch.equal(a, b)
