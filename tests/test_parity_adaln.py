"""GPU parity of the adaLN-modulated QKV projection entry points against the fp64 oracle on the same
seeded inputs (bf16 tensors taken at their exact values).

Tolerances, from the arithmetic: h is rounded to bf16 (relative 2^-9 per element) and multiplies the
bf16 weights with fp32 accumulation, and q, k, v are rounded to bf16 once more, so the outputs carry
about 2 x 2^-9 / sqrt(3) ~ 2.3e-3 relative error: forward relative L2 <= 5e-3 and max abs <= 2e-2
(outputs of magnitude ~0.6, at most ~3), as for the attention. Gradients: relative L2 <= 1e-2 each
(dx adds its own bf16 rounding; dW, dmod and dbias are fp32 sums of exact or once-rounded terms)."""
import numpy as np
import pytest
import torch

from diffusion_transformer_joint_amd import adaln
from diffusion_transformer_joint_amd.inputs import ADALN_WORKLOADS, make_adaln_inputs, make_workload_adaln_inputs
from oracle import adaln_qkv_fwd_bwd

pytestmark = pytest.mark.gpu

FWD_REL, FWD_ABS, BWD_REL = 5e-3, 2e-2, 1e-2


def say(msg):
    print(msg, flush=True)


def f64(t):
    return t.double().cpu().numpy()


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def run_gpu(inp, bias=True, need_dbias=True):
    dev = torch.device("cuda:0")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in ("x", "mod", "w", "bias", "dq", "dk", "dv")}
    q, k, v, ws = adaln.adaln_qkv_forward(d["x"], d["mod"], d["w"], d["bias"] if bias else None, inp["eps"])
    dx, dmod, dw, db = adaln.adaln_qkv_backward(d["x"], d["mod"], d["w"], d["dq"], d["dk"], d["dv"], ws,
                                                need_dbias=need_dbias)
    torch.cuda.synchronize()
    out = []
    for s in range(2):
        r = dict(q=f64(q[s]), k=f64(k[s]), v=f64(v[s]), dx=f64(dx[s]), dmod=f64(dmod[s]), dw=f64(dw[s]))
        if need_dbias:
            r["dbias"] = f64(db[s])
        out.append(r)
    return out


def run_oracle(inp, s, bias=True, samples=None):
    sl = slice(None) if samples is None else samples
    x = f64(inp["x"][s])[sl]
    B, n, C = x.shape
    g = lambda key: f64(inp[key][s])[sl].reshape(B, n, 1, C)
    return adaln_qkv_fwd_bwd(x, f64(inp["mod"][s])[sl], f64(inp["w"][s]), f64(inp["bias"][s]) if bias else None, 1,
                             inp["eps"], g("dq"), g("dk"), g("dv"))


def check(got, ref, tag, keys=("q", "k", "v", "dx", "dmod", "dw", "dbias"), samples=None):
    errs = {}
    for key in keys:
        if key not in got:
            continue
        a = got[key] if samples is None or key in ("dw", "dbias") else got[key][samples]
        b = ref[key]
        a = a.reshape(b.shape)
        errs[key] = rel_l2(a, b)
        if key in ("q", "k", "v"):
            errs[key + "_abs"] = float(np.max(np.abs(a - b))) if a.size else 0.0
    say(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for key, e in errs.items():
        if key.endswith("_abs"):
            assert e <= FWD_ABS, (tag, key, errs)
        elif key in ("q", "k", "v"):
            assert e <= FWD_REL, (tag, key, errs)
        else:
            assert e <= BWD_REL, (tag, key, errs)


SHAPES = [
    # B, n_img, n_txt, C, bias
    (2, 70, 13, 128, True),
    (1, 300, 1, 192, True),     # 3C = 576: a 256-column tile holds the end of q and the start of k
    (3, 64, 0, 64, True),       # no text stream
    (2, 0, 77, 256, True),      # no image stream
    (2, 130, 20, 320, False),   # no bias
    (1, 100, 30, 1152, True),   # 18 heads of 64
    (1, 65, 3, 3072, True),     # the 768 px model's width
]


@pytest.mark.parametrize("B,n_img,n_txt,C,bias", SHAPES)
def test_adaln_shapes(B, n_img, n_txt, C, bias):
    say(f"case: adaln B{B} n_img {n_img} n_txt {n_txt} C{C} bias={bias}, seed 1")
    inp = make_adaln_inputs(B, n_img, n_txt, C, seed=1)
    got = run_gpu(inp, bias=bias)
    for s, n in enumerate((n_img, n_txt)):
        if n:
            check(got[s], run_oracle(inp, s, bias=bias), f"stream {s} B{B} n{n} C{C}")
        else:
            assert got[s]["q"].size == 0 and got[s]["dx"].size == 0
            assert np.all(got[s]["dmod"] == 0) and np.all(got[s]["dw"] == 0) and np.all(got[s]["dbias"] == 0)


def test_adaln_without_bias_gradient():
    say("case: adaln dbias skipped, B2 n_img 40 n_txt 9 C128")
    inp = make_adaln_inputs(2, 40, 9, 128, seed=2)
    got = run_gpu(inp, need_dbias=False)
    for s in range(2):
        check(got[s], run_oracle(inp, s), f"no dbias stream {s}")


def test_adaln_full_mmdit512():
    """The 512 px model's layer (B16, 1024 + 77 tokens, C 768), compared in full."""
    w = ADALN_WORKLOADS["mmdit512"]
    say(f"case: adaln full workload mmdit512 B{w.B} n_img {w.n_img} n_txt {w.n_txt} C{w.C}, seed 0")
    inp = make_workload_adaln_inputs("mmdit512", seed=0)
    got = run_gpu(inp)
    for s in range(2):
        check(got[s], run_oracle(inp, s), f"mmdit512 stream {s}")


def test_adaln_full_mmdit768_sampled():
    """The 768 px model's layer (B4, 2304 + 77 tokens, C 3072): per-sample results of samples 0 and 3
    against the oracle run on those samples alone; the bias gradient against the exact column sums of
    dq, dk, dv; and the weight gradient through the identity <dW, W> + <db, b> = sum(q dq + k dk + v dv)
    (the loss is linear in (W, b)), with q, k, v from the oracle."""
    w = ADALN_WORKLOADS["mmdit768"]
    say(f"case: adaln full workload mmdit768 B{w.B} n_img {w.n_img} n_txt {w.n_txt} C{w.C}, seed 0")
    inp = make_workload_adaln_inputs("mmdit768", seed=0)
    got = run_gpu(inp)
    for s in range(2):
        for b in (0, w.B - 1):
            ref = run_oracle(inp, s, samples=slice(b, b + 1))
            check(got[s], ref, f"mmdit768 stream {s} sample {b}", keys=("q", "k", "v", "dx"), samples=slice(b, b + 1))
            assert rel_l2(got[s]["dmod"][b], ref["dmod"][0]) <= BWD_REL
        cols = np.concatenate([f64(inp[k][s]).reshape(-1, w.C) for k in ("dq", "dk", "dv")], axis=1).sum(axis=0)
        assert rel_l2(got[s]["dbias"], cols) <= 1e-5
        # Euler identity with the oracle's outputs: sum over tokens of y . dy, y = h W^T + b
        x = f64(inp["x"][s])
        mean = x.mean(axis=-1, keepdims=True)
        xh = (x - mean) / np.sqrt(((x - mean) ** 2).mean(axis=-1, keepdims=True) + inp["eps"])
        mod = f64(inp["mod"][s])
        h = (xh * (1 + mod[:, 1][:, None]) + mod[:, 0][:, None]).reshape(-1, w.C)
        dy = np.concatenate([f64(inp[k][s]).reshape(-1, w.C) for k in ("dq", "dk", "dv")], axis=1)
        bias = f64(inp["bias"][s])
        lhs = np.sum(got[s]["dw"] * f64(inp["w"][s])) + np.sum(got[s]["dbias"] * bias)
        rhs = np.sum((dy.T @ h) * f64(inp["w"][s])) + np.sum(dy.sum(axis=0) * bias)
        say(f"mmdit768 stream {s}: <dW,W>+<db,b> {lhs:.6e} vs {rhs:.6e}")
        assert abs(lhs - rhs) <= 1e-2 * (abs(rhs) + np.linalg.norm(got[s]["dw"]) * np.linalg.norm(f64(inp["w"][s])))


def test_adaln_deterministic_and_autograd():
    say("case: adaln determinism and autograd, B2 n_img 100 n_txt 17 C192")
    inp = make_adaln_inputs(2, 100, 17, 192, seed=3)
    dev = torch.device("cuda:0")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in ("x", "mod", "w", "bias", "dq", "dk", "dv")}
    leaf = {k: tuple(t.clone().requires_grad_(True) for t in d[k]) for k in ("x", "mod", "w", "bias")}
    q, k, v = adaln.adaln_qkv(leaf["x"], leaf["mod"], leaf["w"], leaf["bias"], inp["eps"], heads=3)
    loss = sum((t.float() * g.float().reshape(t.shape)).sum() for tt, gg in ((q, d["dq"]), (k, d["dk"]), (v, d["dv"]))
               for t, g in zip(tt, gg))
    loss.backward()
    q2, k2, v2, ws = adaln.adaln_qkv_forward(d["x"], d["mod"], d["w"], d["bias"], inp["eps"], heads=3)
    r1 = adaln.adaln_qkv_backward(d["x"], d["mod"], d["w"], d["dq"], d["dk"], d["dv"], ws)
    r1 = [tuple(t.clone() for t in pair) for pair in r1]
    r2 = adaln.adaln_qkv_backward(d["x"], d["mod"], d["w"], d["dq"], d["dk"], d["dv"], ws)
    torch.cuda.synchronize()
    for a, b in zip((q, k, v), (q2, k2, v2)):
        for s in range(2):
            assert torch.equal(a[s].detach(), b[s]) and a[s].shape == (2, (100, 17)[s], 3, 64)
    for p1, p2 in zip(r1, r2):
        for a, b in zip(p1, p2):
            assert torch.equal(a, b)
    dx, dmod, dw, db = r1
    for s in range(2):
        assert torch.equal(leaf["x"][s].grad, dx[s]) and torch.equal(leaf["mod"][s].grad, dmod[s])
        assert torch.equal(leaf["w"][s].grad, dw[s].to(torch.bfloat16)) and torch.equal(leaf["bias"][s].grad, db[s])


def test_adaln_events_and_reused_workspaces():
    """Stage events on every kernel leave the outputs bitwise unchanged, and a smaller problem run in
    the workspaces of a larger one matches the oracle."""
    from diffusion_transformer_joint_amd import _lib
    say("case: adaln events, B2 n_img 90 n_txt 21 C192; then B1 n_img 33 n_txt 5 in the same workspaces")
    dev = torch.device("cuda:0")
    inp = make_adaln_inputs(2, 90, 21, 192, seed=8)
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in ("x", "mod", "w", "bias", "dq", "dk", "dv")}
    q, k, v, ws = adaln.adaln_qkv_forward(d["x"], d["mod"], d["w"], d["bias"], inp["eps"])
    g = adaln.adaln_qkv_backward(d["x"], d["mod"], d["w"], d["dq"], d["dk"], d["dv"], ws)
    g = tuple(tuple(t.clone() for t in pair) for pair in g)
    ev_f = [torch.cuda.Event(enable_timing=True) for _ in _lib.ADALN_FWD_STAGES]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in _lib.ADALN_BWD_STAGES]
    q2, k2, v2, ws2 = adaln.adaln_qkv_forward(d["x"], d["mod"], d["w"], d["bias"], inp["eps"], events=ev_f)
    g2 = adaln.adaln_qkv_backward(d["x"], d["mod"], d["w"], d["dq"], d["dk"], d["dv"], ws2, events=ev_b)
    torch.cuda.synchronize()
    for s in range(2):
        for a, b in ((q, q2), (k, k2), (v, v2)) + tuple(zip(g, g2)):
            assert torch.equal(a[s], b[s])
    small = make_adaln_inputs(1, 33, 5, 192, seed=9)
    ds = {k: tuple(t.to(dev).contiguous() for t in small[k]) for k in ("x", "mod", "w", "bias", "dq", "dk", "dv")}
    bws = torch.empty(adaln.bwd_workspace_bytes(2, 90, 21, 192), dtype=torch.uint8, device=dev)
    qs, ks, vs, _ = adaln.adaln_qkv_forward(ds["x"], ds["mod"], ds["w"], ds["bias"], small["eps"], workspace=ws)
    dx, dmod, dw, db = adaln.adaln_qkv_backward(ds["x"], ds["mod"], ds["w"], ds["dq"], ds["dk"], ds["dv"], ws,
                                                workspace=bws)
    torch.cuda.synchronize()
    for s in range(2):
        got = dict(q=f64(qs[s]), k=f64(ks[s]), v=f64(vs[s]), dx=f64(dx[s]), dmod=f64(dmod[s]), dw=f64(dw[s]),
                   dbias=f64(db[s]))
        check(got, run_oracle(small, s), f"reused workspaces, stream {s}")
