"""Write the oracle's gain gradients for the full-size workloads to tests/golden/dgains_<name>.json.

The gain gradient sums over every (batch, head) pair, so at full size it is the one output the
parity tests cannot recompute from a few sampled pairs in seconds. This script computes it with the
fp64 oracle only (inputs from the seeded workload generator, seed 0) and stores it; the GPU tests
compare against the stored values.

    python tests/golden/make_golden.py [workload ...]

A name "streams:<workload>" stores the two-stream form instead (dgains_streams_<workload>.json): the
same seed-0 workload split into image and text tensors with a QK-norm gain pair per stream. A
packed variable-length workload name (varlen_*) stores that workload's gain gradients. A name
"window:<workload>" stores the workload under a local window of 256 keys each way
(dgains_window_<workload>.json).
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from diffusion_transformer_joint_amd.inputs import make_inputs, make_stream_inputs, make_varlen_inputs  # noqa: E402
from oracle import attention_fwd_bwd, streams_fwd_bwd, varlen_fwd_bwd  # noqa: E402

FULL = ["mmdit512", "dit256", "mmdit768", "ragged", "streams:mmdit512", "varlen_multires", "varlen_ragged",
        "window:mmdit512"]
WINDOW = (256, 256)


def f64(t):
    import torch
    return t.to(torch.float64).numpy()


def streams(name):
    t0 = time.time()
    inp = make_stream_inputs(name, seed=0)
    vl = None if inp["valid_len"] is None else inp["valid_len"].tolist()
    pair = lambda key: (f64(inp[key][0]), f64(inp[key][1]))
    r = streams_fwd_bwd(pair("q"), pair("k"), pair("v"), inp["gains"].double().numpy(), pair("dout"), vl,
                        inp["scale"], inp["eps"])
    w = inp["workload"]
    rec = dict(workload=name, form="two-stream", seed=0, B=w.B, n_img=w.n_img, n_txt=w.n_txt, H=w.H, D=w.D,
               valid_len=vl, scale=inp["scale"], eps=inp["eps"],
               source="oracle/jattn_oracle.py streams_fwd_bwd, fp64, all pairs",
               dgains=np.asarray(r["dgains"]).tolist())
    with open(os.path.join(HERE, f"dgains_streams_{name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(f"streams:{name}: {time.time() - t0:.1f} s", flush=True)


def varlen(name):
    t0 = time.time()
    inp = make_varlen_inputs(name, seed=0)
    r = varlen_fwd_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["gains"].double().numpy(), f64(inp["dout"]),
                       inp["cu_seqlens"].tolist(), inp["scale"], inp["eps"])
    w = inp["workload"]
    rec = dict(workload=name, form="packed variable-length", seed=0, B=w.B, H=w.H, D=w.D, lengths=inp["lengths"],
               scale=inp["scale"], eps=inp["eps"], source="oracle/jattn_oracle.py varlen_fwd_bwd, fp64, all sequences",
               dgains=np.asarray(r["dgains"]).tolist())
    with open(os.path.join(HERE, f"dgains_{name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(f"{name}: {time.time() - t0:.1f} s", flush=True)


def windowed(name):
    t0 = time.time()
    inp = make_inputs(name, seed=0)
    vl = None if inp["valid_len"] is None else inp["valid_len"].tolist()
    r = attention_fwd_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["gains"].double().numpy(),
                          f64(inp["dout"]), vl, inp["scale"], inp["eps"], window=WINDOW)
    w = inp["workload"]
    rec = dict(workload=name, form="local window", window=list(WINDOW), seed=0, B=w.B, L=w.L, H=w.H, D=w.D,
               valid_len=vl, scale=inp["scale"], eps=inp["eps"],
               source="oracle/jattn_oracle.py attention_fwd_bwd(window=...), fp64, all pairs",
               dgains=np.asarray(r["dgains"]).tolist())
    with open(os.path.join(HERE, f"dgains_window_{name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(f"window:{name}: {time.time() - t0:.1f} s", flush=True)


def main(names):
    for name in names:
        if name.startswith("window:"):
            windowed(name.split(":", 1)[1])
            continue
        if name.startswith("streams:"):
            streams(name.split(":", 1)[1])
            continue
        if name.startswith("varlen_"):
            varlen(name)
            continue
        t0 = time.time()
        inp = make_inputs(name, seed=0)
        vl = None if inp["valid_len"] is None else inp["valid_len"].tolist()
        r = attention_fwd_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["gains"].double().numpy(),
                              f64(inp["dout"]), vl, inp["scale"], inp["eps"])
        w = inp["workload"]
        rec = dict(workload=name, seed=0, B=w.B, L=w.L, H=w.H, D=w.D, valid_len=vl, scale=inp["scale"],
                   eps=inp["eps"], source="oracle/jattn_oracle.py attention_fwd_bwd, fp64, all pairs",
                   dgains=np.asarray(r["dgains"]).tolist(),
                   out_sq_sum=float(np.sum(r["out"] ** 2)))
        with open(os.path.join(HERE, f"dgains_{name}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(f"{name}: {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or FULL)
