"""GPU parity of the MLP-block entry points (fc, adaLN, SwiGLU, one residual) against the fp64 oracle on
the same seeded inputs (bf16 tensors at their exact values).

Tolerances, from the arithmetic: the block rounds four intermediates to bf16 (z, u, [a|g] or hid, and
out), each a relative 2^-9 (2e-3) per element, and the LayerNorm rescales z's rounding by 1/std(z). The
block's own contribution y is taken from a second forward call with x = 0 (out = y, rounded relative
to y; out - x would carry out's rounding relative to |x|, ten times |y| here) and compared with
relative L2 <= 1e-2; out itself with the forward bound of the attention (5e-3 relative L2, 2e-2 max
abs). Gradients: relative L2 <= 1e-2 each (fp32 sums of once-rounded terms; do passes through two more
bf16 intermediates, d[a|g] and dz, and still measures about 4e-3)."""
import numpy as np
import pytest
import torch

from diffusion_transformer_joint_amd import _lib, mlp
from diffusion_transformer_joint_amd.inputs import MLP_WORKLOADS, make_mlp_inputs, make_workload_mlp_inputs
from oracle import mlp_fwd_bwd

pytestmark = pytest.mark.gpu

OUT_REL, OUT_ABS, Y_REL, GRAD_REL, DO_REL = 5e-3, 2e-2, 1e-2, 1e-2, 1e-2
KEYS = ("o", "x", "mod", "wfc", "bfc", "w12", "b12", "w2", "b2", "dout")


def say(msg):
    print(msg, flush=True)


def f64(t):
    return t.double().cpu().numpy()


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def run_gpu(inp, bias=True):
    dev = torch.device("cuda:0")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in KEYS}
    b = lambda k: d[k] if bias else None
    out, ws = mlp.mlp_forward(d["o"], d["x"], d["mod"], d["wfc"], d["w12"], d["w2"], b("bfc"), b("b12"), b("b2"),
                              inp["eps"])
    g = mlp.mlp_backward(d["o"], d["mod"], d["wfc"], d["w12"], d["w2"], d["dout"], ws)
    zero = tuple(torch.zeros_like(t) for t in d["x"])
    y, _ = mlp.mlp_forward(d["o"], zero, d["mod"], d["wfc"], d["w12"], d["w2"], b("bfc"), b("b12"), b("b2"), inp["eps"])
    torch.cuda.synchronize()
    res = []
    for s in range(2):
        r = {k: f64(v[s]) for k, v in g.items()}
        r["out"], r["y"] = f64(out[s]), f64(y[s])
        res.append(r)
    return res


def run_oracle(inp, s, bias=True, samples=slice(None), tokens=slice(None)):
    t = lambda k: f64(inp[k][s])[samples][:, tokens]
    w = lambda k: f64(inp[k][s])
    bb = lambda k: f64(inp[k][s]) if bias else None
    return mlp_fwd_bwd(t("o"), t("x"), f64(inp["mod"][s])[samples], w("wfc"), bb("bfc"), w("w12"), bb("b12"), w("w2"),
                       bb("b2"), inp["eps"], t("dout"))


def check(got, ref, inp, s, tag, keys=None, samples=slice(None), tokens=slice(None)):
    errs = {}
    go = got["out"][samples][:, tokens]
    errs["out"], errs["out_abs"] = rel_l2(go, ref["out"]), float(np.max(np.abs(go - ref["out"]))) if go.size else 0.0
    errs["y"] = rel_l2(got["y"][samples][:, tokens], ref["y"])
    errs["do"] = rel_l2(got["do"][samples][:, tokens], ref["do"])
    for k in keys if keys is not None else ("dmod", "dwfc", "dbfc", "dw12", "db12", "dw2", "db2"):
        a = got[k][samples] if k == "dmod" else got[k]
        errs[k] = rel_l2(a, ref[k])
    say(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["out"] <= OUT_REL and errs["out_abs"] <= OUT_ABS, (tag, errs)
    assert errs["y"] <= Y_REL, (tag, errs)
    assert errs["do"] <= DO_REL, (tag, errs)
    for k, e in errs.items():
        if k.startswith("d") and k != "do":
            assert e <= GRAD_REL, (tag, k, errs)


SHAPES = [
    # B, n_img, n_txt, C, F, bias
    (2, 70, 13, 128, 256, True),
    (1, 300, 1, 192, 320, True),     # F = 320: the last 128-column tile of W1 and W3 is half full
    (3, 64, 0, 64, 64, True),        # no text stream
    (2, 0, 77, 256, 512, True),      # no image stream
    (2, 130, 20, 320, 384, False),   # no biases
]


@pytest.mark.parametrize("B,n_img,n_txt,C,F,bias", SHAPES)
def test_mlp_shapes(B, n_img, n_txt, C, F, bias):
    say(f"case: mlp B{B} n_img {n_img} n_txt {n_txt} C{C} F{F} bias={bias}, seed 1")
    inp = make_mlp_inputs(B, n_img, n_txt, C, F, seed=1)
    got = run_gpu(inp, bias=bias)
    for s, n in enumerate((n_img, n_txt)):
        if n:
            check(got[s], run_oracle(inp, s, bias=bias), inp, s, f"stream {s} n{n} C{C} F{F}")
        else:
            assert got[s]["out"].size == 0 and got[s]["do"].size == 0
            for k in ("dmod", "dwfc", "dbfc", "dw12", "db12", "dw2", "db2"):
                assert np.all(got[s][k] == 0), k


def test_mlp_full_mmdit512():
    """The 512 px model's layer (B16, 1024 + 77 tokens, C 768, F 2048), compared in full."""
    w = MLP_WORKLOADS["mmdit512"]
    say(f"case: mlp full workload mmdit512 B{w.B} n_img {w.n_img} n_txt {w.n_txt} C{w.C} F{w.F}, seed 0")
    inp = make_workload_mlp_inputs("mmdit512", seed=0)
    got = run_gpu(inp)
    for s in range(2):
        check(got[s], run_oracle(inp, s), inp, s, f"mmdit512 stream {s}")


def test_mlp_full_mmdit768_sampled():
    """The 768 px model's layer (B4, 2304 + 77 tokens, C 3072, F 8192): the text stream against the full
    oracle; out and do of 96 image tokens of samples 0 and 3 against the oracle run on those tokens (the
    block is per token apart from its sums); the image stream's bias gradients against the exact column
    sums; its (W2, b2) gradients through the identity <dW2, W2> + <db2, b2> = sum(dout * y)."""
    w = MLP_WORKLOADS["mmdit768"]
    say(f"case: mlp full workload mmdit768 B{w.B} n_img {w.n_img} n_txt {w.n_txt} C{w.C} F{w.F}, seed 0")
    inp = make_workload_mlp_inputs("mmdit768", seed=0)
    got = run_gpu(inp)
    check(got[1], run_oracle(inp, 1), inp, 1, "mmdit768 text stream")
    tok = slice(0, w.n_img, w.n_img // 96)
    for b in (0, w.B - 1):
        ref = run_oracle(inp, 0, samples=slice(b, b + 1), tokens=tok)
        check(got[0], ref, inp, 0, f"mmdit768 image sample {b}, 96 tokens", keys=(), samples=slice(b, b + 1),
              tokens=tok)
    dout = f64(inp["dout"][0]).reshape(-1, w.C)
    assert rel_l2(got[0]["db2"], dout.sum(axis=0)) <= 1e-5
    y = got[0]["y"]
    lhs = np.sum(got[0]["dw2"] * f64(inp["w2"][0])) + np.sum(got[0]["db2"] * f64(inp["b2"][0]))
    rhs = float(np.sum(f64(inp["dout"][0]) * y))
    say(f"mmdit768 image: <dW2,W2>+<db2,b2> {lhs:.6e} vs {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-2 * np.linalg.norm(dout) * np.linalg.norm(y)


def test_mlp_deterministic_and_autograd():
    say("case: mlp determinism and autograd, B2 n_img 100 n_txt 17 C192 F256")
    inp = make_mlp_inputs(2, 100, 17, 192, 256, seed=3)
    dev = torch.device("cuda:0")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in KEYS}
    leaf = {k: tuple(t.clone().requires_grad_(True) for t in d[k]) for k in KEYS if k != "dout"}
    out = mlp.mlp_block(leaf["o"], leaf["x"], leaf["mod"], leaf["wfc"], leaf["w12"], leaf["w2"], leaf["bfc"],
                        leaf["b12"], leaf["b2"], inp["eps"])
    sum((t.float() * g.float()).sum() for t, g in zip(out, d["dout"])).backward()
    out2, ws = mlp.mlp_forward(d["o"], d["x"], d["mod"], d["wfc"], d["w12"], d["w2"], d["bfc"], d["b12"], d["b2"],
                               inp["eps"])
    g1 = mlp.mlp_backward(d["o"], d["mod"], d["wfc"], d["w12"], d["w2"], d["dout"], ws)
    g1 = {k: tuple(t.clone() for t in v) for k, v in g1.items()}
    g2 = mlp.mlp_backward(d["o"], d["mod"], d["wfc"], d["w12"], d["w2"], d["dout"], ws)
    torch.cuda.synchronize()
    for s in range(2):
        assert torch.equal(out[s].detach(), out2[s])
        for k in g1:
            assert torch.equal(g1[k][s], g2[k][s]), k
        assert torch.equal(leaf["o"][s].grad, g1["do"][s]) and torch.equal(leaf["x"][s].grad, d["dout"][s])
        assert torch.equal(leaf["mod"][s].grad, g1["dmod"][s])
        for k, gk in (("wfc", "dwfc"), ("w12", "dw12"), ("w2", "dw2")):
            assert torch.equal(leaf[k][s].grad, g1[gk][s].to(torch.bfloat16)), k
        for k, gk in (("bfc", "dbfc"), ("b12", "db12"), ("b2", "db2")):
            assert torch.equal(leaf[k][s].grad, g1[gk][s]), k


def test_mlp_options_do_not_change_results():
    """No bias gradients (NULL pointers), stage events on every kernel, and caller workspaces reused
    from a larger call leave every written output bitwise equal to the plain call."""
    say("case: mlp options, B2 n_img 96 n_txt 33 C128 F192 (then B1 n_img 40 n_txt 9 into the same workspaces)")
    dev = torch.device("cuda:0")
    inp = make_mlp_inputs(2, 96, 33, 128, 192, seed=5)
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in KEYS}
    fa = lambda **kw: mlp.mlp_forward(d["o"], d["x"], d["mod"], d["wfc"], d["w12"], d["w2"], d["bfc"], d["b12"],
                                      d["b2"], inp["eps"], **kw)
    ba = lambda ws, **kw: mlp.mlp_backward(d["o"], d["mod"], d["wfc"], d["w12"], d["w2"], d["dout"], ws, **kw)
    out, ws = fa()
    ref = ba(ws)
    ref = {k: tuple(t.clone() for t in v) for k, v in ref.items()}
    ev_f = [torch.cuda.Event(enable_timing=True) for _ in range(len(_lib.MLP_FWD_STAGES))]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(len(_lib.MLP_BWD_STAGES))]
    out_e, ws_e = fa(events=ev_f)
    g_e = ba(ws_e, events=ev_b)
    g_n = ba(ws, need_dbias=False)
    torch.cuda.synchronize()
    for s in range(2):
        assert torch.equal(out_e[s], out[s])
        for k in ref:
            assert torch.equal(g_e[k][s], ref[k][s]), k
            if k not in ("dbfc", "db12", "db2"):
                assert torch.equal(g_n[k][s], ref[k][s]), k
    assert not any(k in g_n for k in ("dbfc", "db12", "db2"))
    # a smaller problem into the first call's (larger) workspaces, against the oracle
    small = make_mlp_inputs(1, 40, 9, 128, 192, seed=6)
    ds = {k: tuple(t.to(dev).contiguous() for t in small[k]) for k in KEYS}
    fws_big = ws
    bws_big = torch.empty(mlp.bwd_workspace_bytes(2, 96, 33, 128, 192), dtype=torch.uint8, device=dev)
    out_s, _ = mlp.mlp_forward(ds["o"], ds["x"], ds["mod"], ds["wfc"], ds["w12"], ds["w2"], ds["bfc"], ds["b12"],
                               ds["b2"], small["eps"], workspace=fws_big)
    g_s = mlp.mlp_backward(ds["o"], ds["mod"], ds["wfc"], ds["w12"], ds["w2"], ds["dout"], fws_big, workspace=bws_big)
    zero = tuple(torch.zeros_like(t) for t in ds["x"])
    y_s, _ = mlp.mlp_forward(ds["o"], zero, ds["mod"], ds["wfc"], ds["w12"], ds["w2"], ds["bfc"], ds["b12"], ds["b2"],
                             small["eps"])
    torch.cuda.synchronize()
    for s in range(2):
        got = {k: f64(v[s]) for k, v in g_s.items()}
        got["out"], got["y"] = f64(out_s[s]), f64(y_s[s])
        check(got, run_oracle(small, s), small, s, f"reused workspaces, stream {s}")


def test_mlp_wide_layer_partial_tiles():
    """C = 1152 (18 heads of 64) and F = 3136 (not a multiple of 128: the last W1/W3 column tile is half
    full), 2 samples of 250 + 29 tokens, against the full oracle."""
    say("case: mlp B2 n_img 250 n_txt 29 C1152 F3136, seed 7")
    inp = make_mlp_inputs(2, 250, 29, 1152, 3136, seed=7)
    got = run_gpu(inp)
    for s in range(2):
        check(got[s], run_oracle(inp, s), inp, s, f"wide layer stream {s}")
