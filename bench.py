"""Benchmark: joint-attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mmdit512] [--no-cpu-baseline]
                    [--calibrate-copy] [--calibrate-busy] [--flush-mall]
                    [--variant joint|streams|varlen|window|adaln|mlp]

A step is one forward (jattn_fwd) plus one backward (jattn_bwd) over the whole batch of the workload,
inputs resident in HBM. Prints one JSON line. Before the --warmup steps a pre-roll runs steps in
windows of 10 until the last three windows agree within 2 % (reported as `preroll`), so the timed
region starts at steady clocks however few warm-up steps are asked for. The throughput is algorithmic TFLOP/s:
4*B*H*L*L*D for the forward (valid keys only for ragged workloads) and 2.5x that for the backward.

Joint-variant lines also carry `hbm` (the step's algorithmic HBM bytes, 8BLHD + 4BHL forward and
16BLHD + 8BHL backward, and the rate they imply against 8 TB/s) and `per_step` (median and minimum of
the fwd, bwd and fwd+bwd times over the breakdown pass). --flush-mall adds `hbm.cold`: the same step
timed with 512 MiB written before each step, so that no operand is left in the 256 MB Infinity Cache.
--calibrate-busy runs the saturating probe kernels first (see include/jattn_diag.h).

--variant streams times the two-stream entry points instead (image and text tensors of the same
workload, a QK-norm gain pair per stream: jattn_fwd_streams + jattn_bwd_streams), and beside them the
step they replace: concatenating the stream tensors, the joint forward and backward, and splitting
the outputs and gradients back (`concat_split`).

--variant window times the local-window entry points (jattn_fwd_window + jattn_bwd_window, window
--window LEFT RIGHT, default 256 256; FLOPs over the (query, key) pairs the window allows) and beside
them full attention on the same inputs (`full`).

--variant varlen (with --workload varlen_multires or varlen_ragged) times the packed variable-length
entry points (jattn_fwd_varlen + jattn_bwd_varlen; FLOPs over each sequence's own query-key pairs),
and beside them the same sequences padded to the longest one through the joint entry points with a
key mask (`padded`).

--variant adaln (with --workload mmdit512 or mmdit768) times the adaLN-modulated QKV projection of
both streams of a layer (jattn_adaln_qkv_fwd + jattn_adaln_qkv_bwd; FLOPs of its three GEMMs,
2 T C 3C each for T tokens of width C), and beside it the same step written as torch's LayerNorm,
modulation and Linear with autograd (`torch_unfused`).

--variant mlp (with --workload mmdit512 or mmdit768) times the MLP block after the attention (fc,
adaLN, SwiGLU, one residual; jattn_mlp_fwd + jattn_mlp_bwd over both streams; FLOPs of its GEMMs,
2 T (C^2 + 3 C F) forward and twice that backward), and beside it the same step in torch ops
(`torch_unfused`).
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attn fwd+bwd TFLOP/s @ B16 L1101 H12 D64 bf16; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mmdit512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--variant", choices=("joint", "streams", "varlen", "window", "adaln", "mlp"), default="joint")
    ap.add_argument("--window", type=int, nargs=2, default=(256, 256), metavar=("LEFT", "RIGHT"))
    ap.add_argument("--flush-mall", action="store_true",
                    help="joint variant: also time steps with a 512 MiB write between them (more than the "
                         "256 MB Infinity Cache), so every step starts with cold caches")
    ap.add_argument("--calibrate-busy", action="store_true",
                    help="first run the library's saturating MFMA and FMA probe kernels (about 1 ms each): "
                         "under rocprofv3 --pmc their busy-counter readings are the full-scale values")
    ap.add_argument("--probe-dq-accumulation", action="store_true",
                    help="instead of the step: time the memory traffic a key-parallel backward would need to "
                         "accumulate dQ across key blocks (fp32 atomics, or partial sums and their reduction; "
                         "include/jattn_diag.h) at the workload's shape, beside the dq kernel it would replace")
    ap.add_argument("--probe-tile", action="store_true",
                    help="time the dk/dv tile's dependency structure (jattn_probe_tile) with its operands in "
                         "registers or LDS, the LDS read rates (jattn_probe_lds_read), the MFMA / FMA / exp2 "
                         "issue rates (jattn_probe_issue) and the forward tile's wave schedules "
                         "(jattn_probe_pingpong); prints one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy 512 MiB device-to-device three times: under rocprofv3 --pmc its "
                         "FETCH_SIZE / WRITE_SIZE give the counters' scale for a known byte count")
    return ap.parse_args()


COPY_BYTES = 512 << 20


# Device sources (kernels, their launchers and device headers) behind each entry-point family.
KERNEL_SOURCES = {
    "attention": ("jattn_device.h", "jattn_launch.h", "jattn_prenorm.hip", "jattn_fwd.hip", "jattn_bwd.hip",
                  "jattn_bwd_kernels.h", "jattn_bwd_wide.hip"),
    "projection": ("jattn_device.h", "adaln_launch.h", "adaln_qkv.hip"),
}


def kernel_sources_digest(variant="joint"):
    """sha256 over the device sources of the kernels a variant runs: ties stored counter readings to a
    kernel version (a change to those sources voids them; host-side API files do not)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "diffusion_transformer_joint_amd", "csrc")
    for name in KERNEL_SOURCES["projection" if variant in ("adaln", "mlp") else "attention"]:
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload, kernel, variant="joint", window=None):
    """HBM bytes per launch of `kernel` from the committed counter summary of this workload (and entry
    point variant, and window for the local-window form), or None when there is none, it was read with
    another window, or the library sources changed since the counters were read."""
    suffix = "" if variant in ("joint", "varlen") else f"_{variant}"  # (varlen workloads are named so)
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}{suffix}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    rec = json.loads(text[start + 7:text.index("```", start + 7)])
    if rec.get("source_sha256") != kernel_sources_digest(variant):
        return None
    if window is not None and rec.get("window") != list(window):
        return None
    ent = rec.get("kernels", {}).get(kernel)
    return None if ent is None else ent["hbm_bytes_per_launch"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the op shards with no "
              "communication: each GPU runs its own micro-batch).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_busy:
        run_busy_probes(torch)
    if args.probe_dq_accumulation:
        return probe_dq_accumulation(args, torch)
    if args.probe_tile:
        return probe_tile(torch)
    if args.variant == "adaln":
        return bench_adaln(args, torch)
    if args.variant == "mlp":
        return bench_mlp(args, torch)

    from diffusion_transformer_joint_amd import _lib
    from diffusion_transformer_joint_amd.inputs import (VARLEN_WORKLOADS, WORKLOADS, flops, make_inputs,
                                                        make_stream_inputs, make_varlen_inputs, varlen_flops)

    streams, varlen, windowed = args.variant == "streams", args.variant == "varlen", args.variant == "window"
    if varlen and args.workload not in VARLEN_WORKLOADS:
        args.workload = "varlen_multires"
    if varlen:
        w = VARLEN_WORKLOADS[args.workload]
        inp = make_varlen_inputs(args.workload, seed=0)
        B, H, D, L = w.B, w.H, w.D, inp["max_seqlen"]
        total = sum(inp["lengths"])
    else:
        w = WORKLOADS[args.workload]
        B, L, H, D = w.B, w.L, w.H, w.D
        inp = make_stream_inputs(args.workload, seed=0) if streams else make_inputs(args.workload, seed=0)
    dev = torch.device("cuda:0")
    gains = inp["gains"].to(dev)
    vl = None if inp.get("valid_len") is None else inp["valid_len"].to(dev)
    lse = torch.empty(total * H if varlen else B * H * L, dtype=torch.float32, device=dev)
    lib = _lib.load()
    if varlen:
        ws_bytes = int(lib.jattn_varlen_bwd_workspace_bytes(B, L, total, H, D))
        fws_bytes = int(lib.jattn_varlen_fwd_workspace_bytes(B, L, total, H, D))
    else:
        ws_bytes = int(lib.jattn_bwd_workspace_bytes(B, L, H, D))
        fws_bytes = int(lib.jattn_fwd_workspace_bytes(B, L, H, D))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    scale, eps = ctypes.c_float(inp["scale"]), ctypes.c_float(inp["eps"])
    vlp = None if vl is None else vl.data_ptr()
    if varlen:
        q, k, v, dout = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
        cu = inp["cu_seqlens"].to(dev)
        out = torch.empty_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dg = torch.empty(2, D, dtype=torch.float32, device=dev)
        fwd_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), cu.data_ptr(), B, L, total, H, D,
                    scale, eps, out.data_ptr(), lse.data_ptr(), fws.data_ptr(), fws_bytes)
        bwd_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), cu.data_ptr(), out.data_ptr(),
                    lse.data_ptr(), dout.data_ptr(), B, L, total, H, D, scale, eps, dq.data_ptr(), dk.data_ptr(),
                    dv.data_ptr(), dg.data_ptr(), ws.data_ptr(), ws_bytes, fws.data_ptr())

        def fwd(events=None, n=len(_lib.FWD_STAGES)):
            _lib.check("jattn_fwd_varlen", lib.jattn_fwd_varlen(*fwd_args, events, 0 if events is None else n, sp))

        def bwd(events=None, n=len(_lib.BWD_STAGES)):
            _lib.check("jattn_bwd_varlen", lib.jattn_bwd_varlen(*bwd_args, events, 0 if events is None else n, sp))
    elif not streams:
        q, k, v, dout = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
        out = torch.empty_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dg = torch.empty(2, D, dtype=torch.float32, device=dev)
        fwd_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), vlp, B, L, H, D, scale, eps,
                    out.data_ptr(), lse.data_ptr(), fws.data_ptr(), fws_bytes, sp)
        bwd_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), vlp, out.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), B, L, H, D, scale, eps, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    dg.data_ptr(), ws.data_ptr(), ws_bytes, fws.data_ptr(), sp)

        if windowed:
            wl, wr = args.window
            fwd_w = fwd_args[:11] + (wl, wr) + fwd_args[11:-1]
            bwd_w = bwd_args[:14] + (wl, wr) + bwd_args[14:-1]

            def fwd(events=None, n=len(_lib.FWD_STAGES)):
                _lib.check("jattn_fwd_window", lib.jattn_fwd_window(*fwd_w, events, 0 if events is None else n, sp))

            def bwd(events=None, n=len(_lib.BWD_STAGES)):
                _lib.check("jattn_bwd_window", lib.jattn_bwd_window(*bwd_w, events, 0 if events is None else n, sp))
        else:
            def fwd(events=None, n=len(_lib.FWD_STAGES)):
                if events is None:
                    _lib.check("jattn_fwd", lib.jattn_fwd(*fwd_args))
                else:
                    _lib.check("jattn_fwd_ex", lib.jattn_fwd_ex(*fwd_args[:-1], events, n, sp))

            def bwd(events=None, n=len(_lib.BWD_STAGES)):
                if events is None:
                    _lib.check("jattn_bwd", lib.jattn_bwd(*bwd_args))
                else:
                    _lib.check("jattn_bwd_ex", lib.jattn_bwd_ex(*bwd_args[:-1], events, n, sp))
    else:
        part = lambda t: tuple(x.to(dev) for x in t)
        q, k, v, dout = (part(inp[n]) for n in ("q", "k", "v", "dout"))
        like = lambda t: (torch.empty_like(t[0]), torch.empty_like(t[1]))
        out, dq, dk, dv = like(q), like(q), like(k), like(v)
        dg = torch.empty(2, 2, D, dtype=torch.float32, device=dev)
        pp = {name: _lib.PtrPair(t[0].data_ptr(), t[1].data_ptr())
              for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk),
                              ("dv", dv))}
        fwd_args = (pp["q"].arg, pp["k"].arg, pp["v"].arg, gains.data_ptr(), vlp, B, w.n_img, w.n_txt, H, D, scale,
                    eps, pp["out"].arg, lse.data_ptr(), fws.data_ptr(), fws_bytes)
        bwd_args = (pp["q"].arg, pp["k"].arg, pp["v"].arg, gains.data_ptr(), vlp, pp["out"].arg, lse.data_ptr(),
                    pp["dout"].arg, B, w.n_img, w.n_txt, H, D, scale, eps, pp["dq"].arg, pp["dk"].arg, pp["dv"].arg,
                    dg.data_ptr(), ws.data_ptr(), ws_bytes, fws.data_ptr())

        def fwd(events=None, n=len(_lib.FWD_STAGES)):
            _lib.check("jattn_fwd_streams", lib.jattn_fwd_streams(*fwd_args, events, 0 if events is None else n, sp))

        def bwd(events=None, n=len(_lib.BWD_STAGES)):
            _lib.check("jattn_bwd_streams", lib.jattn_bwd_streams(*bwd_args, events, 0 if events is None else n, sp))

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # creates the underlying hipEvent_t
        return e

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    pre = preroll(torch, stream, lambda: (fwd(), bwd()), new_event)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    def handle(evs):
        arr = (ctypes.c_void_p * len(evs))(*[None if e is None else e.cuda_event for e in evs])
        return arr, ctypes.cast(arr, ctypes.c_void_p)

    K = args.steps
    # stage labels: the kernels' template instantiations, as a profiler names them
    sflag = "true" if streams else "false"
    targs = f"{D}, {sflag}, {'true' if varlen else 'false'}, {'true' if windowed else 'false'}"
    pargs = targs.rsplit(",", 1)[0]  # the normalisation kernel has no window parameter
    stages = [f"{n}<{pargs}> (fwd)" if n == "prenorm_kernel" else f"{n}<{targs}>" for n in _lib.FWD_STAGES]
    stages += [f"{n}<{pargs}> (bwd)" if n == "prenorm_kernel" else
               (f"{n}<{sflag}>" if n == "dg_reduce_kernel" else f"{n}<{targs}>") for n in _lib.BWD_STAGES]
    nf = len(_lib.FWD_STAGES)
    dq_key, dkdv_key = f"bwd_dq_kernel<{targs}>", f"bwd_dkdv_kernel<{targs}>"

    # Per-kernel breakdown (before the timed region, not part of `value`): every stage event.
    KB = min(K, 50)
    ev0 = [new_event() for _ in range(KB)]
    evb = [[new_event() for _ in stages] for _ in range(KB)]
    fh = [handle(evb[i][:nf]) for i in range(KB)]
    bh = [handle(evb[i][nf:]) for i in range(KB)]
    torch.cuda.synchronize()
    for i in range(KB):
        ev0[i].record(stream)
        fwd(fh[i][1])
        bwd(bh[i][1])
    torch.cuda.synchronize()
    kern_ms = {}
    for j, name in enumerate(stages):
        kern_ms[name] = sum((ev0[i] if j == 0 else evb[i][j - 1]).elapsed_time(evb[i][j]) for i in range(KB)) / KB
    # forward and backward shares from the same (breakdown) pass: the span from the step's start to the
    # forward's last stage event, and from there to the backward's last one
    ms_fwd = sum(ev0[i].elapsed_time(evb[i][nf - 1]) for i in range(KB)) / KB
    ms_bwd = sum(evb[i][nf - 1].elapsed_time(evb[i][-1]) for i in range(KB)) / KB
    # per-step spread from the same pass (events at the step's start, between fwd and bwd, at its end)
    spread = lambda xs: {"median": round(sorted(xs)[len(xs) // 2], 5), "min": round(min(xs), 5)}
    per_step = {"fwd": spread([ev0[i].elapsed_time(evb[i][nf - 1]) for i in range(KB)]),
                "bwd": spread([evb[i][nf - 1].elapsed_time(evb[i][-1]) for i in range(KB)]),
                "fwd+bwd": spread([ev0[i].elapsed_time(evb[i][-1]) for i in range(KB)]),
                "steps": KB, "note": "breakdown pass, every stage event recorded"}

    # Timed region: K steps of forward + backward, with the library's stage events around the kernel
    # that took longest in the breakdown pass only; its live launch duration feeds the roofline. MFMA
    # FLOPs one launch executes per (query, valid key) pair: forward 4D (S, PV); dq kernel 6D (S, dP
    # recomputed, dQ); dk/dv kernel 8D (S, dP, dV, dK).
    per_pair = {f"fwd_kernel<{targs}>": 4 * D, dq_key: 6 * D, dkdv_key: 8 * D}
    dom = max(per_pair, key=lambda k: kern_ms[k])
    ms_step, dom_ms = timed_region(fwd, bwd, stages.index(dom), nf, K, stream, new_event, handle)

    cold = None
    if args.flush_mall and not (streams or varlen or windowed):
        cold = time_cold_steps(torch, stream, fwd, bwd, new_event, KB)

    concat_split = padded = None
    if streams:
        concat_split = time_concat_split(lib, _lib, torch, q, k, v, dout, gains, vl, B, L, H, D, inp, stream, K,
                                         args.warmup)
    if varlen:
        padded = time_padded(lib, _lib, torch, inp, gains, B, L, H, D, stream, K, args.warmup)
    full = None
    if windowed:
        full = time_steps(torch, stream, lambda: (_lib.check("jattn_fwd", lib.jattn_fwd(*fwd_args)),
                                                   _lib.check("jattn_bwd", lib.jattn_bwd(*bwd_args))), K, args.warmup)

    vlist = None if inp.get("valid_len") is None else inp["valid_len"].tolist()
    fl = varlen_flops(inp["lengths"], H, D) if varlen else flops(B, L, H, D, vlist)
    if windowed:
        fl = window_flops(B, L, H, D, vlist, args.window)
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12
    fwd_tflops = fl["fwd"] / (ms_fwd * 1e-3) / 1e12
    bwd_tflops = fl["bwd"] / (ms_bwd * 1e-3) / 1e12
    # Roofline of the dominant kernel
    pairs = fl["fwd"] / (4.0 * H * D)
    achieved = per_pair[dom] * H * pairs / (dom_ms * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(args.workload, dom, args.variant, args.window if windowed else None),
                "flop_per_launch": per_pair[dom] * H * pairs, "avg_launch_ms": round(dom_ms, 5),
                "avg_launch_ms_source": "timed region"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    # (the metric names its shape; the headline workload keeps the headline metric's exact wording)
    metric = METRIC if (args.workload == "mmdit512" and not varlen) else (
        f"joint-attn fwd+bwd TFLOP/s @ {args.workload} B{B} " + ("" if varlen else f"L{L} ") +
        f"H{H} D{D} bf16; % of bf16 MFMA peak")
    res = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": ({"workload": args.workload, "variant": args.variant, "B": B, "H": H, "D": D,
                    "lengths": inp["lengths"], "total": total, "max_seqlen": L, "global_batch": B,
                    "parallelism": "single-gpu"} if varlen else
                   {"workload": args.workload, "variant": args.variant, "B": B, "L": L, "H": H, "D": D,
                    "n_img": w.n_img, "n_txt": w.n_txt, "valid_len": vlist, "global_batch": B, "seq_len": L,
                    "parallelism": "single-gpu"}),
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(ms_fwd, 5),
        "bwd_ms": round(ms_bwd, 5),
        "fwd_bwd_source": "breakdown pass (every stage event recorded; both from the same pass)",
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "gflop_per_step": round(fl["total"] / 1e9, 3),
        "kernel_ms": {k: round(v, 5) for k, v in kern_ms.items()},
        "kernel_ms_timed_region": {dom: round(dom_ms, 5)},
        "per_step": per_step,
        "preroll": pre,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if not varlen:
        # algorithmic HBM bytes of a step: forward reads q, k, v and writes out (8 B L H D) plus the LSE
        # (4 B H L); backward reads q, k, v, out, dout and writes dq, dk, dv (16 B L H D) plus the LSE
        # and row statistics (8 B H L)
        hb = {"fwd": 8.0 * B * L * H * D + 4.0 * B * H * L, "bwd": 16.0 * B * L * H * D + 8.0 * B * H * L}
        hb["total"] = hb["fwd"] + hb["bwd"]
        res["hbm"] = {"algorithmic_bytes": hb["total"], "gbs": round(hb["total"] / (ms_step * 1e-3) / 1e9, 1),
                      "frac_of_8tbs": round(hb["total"] / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "flop_per_byte": round(fl["total"] / hb["total"], 1)}
        if fl.get("fwd_padded") and vlist is not None:
            res["gflop_per_step_dense"] = round(3.5 * fl["fwd_padded"] / 1e9, 3)
        if cold is not None:
            res["hbm"]["cold"] = cold
            res["hbm"]["cold"]["gbs"] = round(hb["total"] / (cold["fwd+bwd"]["median"] * 1e-3) / 1e9, 1)
            res["hbm"]["cold"]["frac_of_8tbs"] = round(res["hbm"]["cold"]["gbs"] / PEAK_HBM_GBS, 4)
    if concat_split is not None:
        res["concat_split"] = concat_split
        res["concat_split"]["speedup"] = round(concat_split["ms_per_step"] / ms_step, 4)
    if windowed:
        res["config"]["window"] = list(args.window)
        res["full"] = {"ms_per_step": round(full, 5), "speedup": round(full / ms_step, 4),
                       "what": "full attention (jattn_fwd + jattn_bwd) on the same inputs"}
    if padded is not None:
        res["padded"] = padded
        res["padded"]["speedup"] = round(padded["ms_per_step"] / ms_step, 4)
    print(json.dumps(res), flush=True)


def preroll(torch, stream, step, new_event, window=10, tol=0.02, min_windows=5, max_windows=100):
    """Run `step` in windows of `window` steps until the last three windows' times agree within `tol`
    (relative), so that the timed region starts at steady clocks whatever --warmup says. Returns the
    record reported as `preroll` in the JSON line."""
    times = []
    for _ in range(max_windows):
        a, b = new_event(), new_event()
        a.record(stream)
        for _ in range(window):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
        last = times[-3:]
        if len(times) >= min_windows and max(last) - min(last) <= tol * min(last):
            break
    last = times[-3:]
    return {"preroll_steps": window * len(times), "preroll_ms": round(sum(times), 3),
            "last_windows_ms_per_step": [round(t / window, 5) for t in last],
            "converged": len(last) == 3 and max(last) - min(last) <= tol * min(last)}


def probe_dq_accumulation(args, torch):
    """Times the dQ accumulation a fused key-parallel backward would need (no attention arithmetic), for
    key blocks of 128, 256 and 384 keys; the dq kernel that recomputes dQ instead is timed by the
    ordinary run of the same workload. Prints one JSON line."""
    from diffusion_transformer_joint_amd import _lib
    from diffusion_transformer_joint_amd.inputs import WORKLOADS
    w = WORKLOADS[args.workload]
    pairs, L, D = w.B * w.H, w.L, w.D
    lib = _lib.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    n = pairs * L * D
    res = {"what": "dQ accumulation across key blocks of a key-parallel backward, memory traffic only",
           "workload": args.workload, "pairs": pairs, "L": L, "D": D, "modes": []}
    for nkb_rows in (128, 256, 384):
        nkb = (L + nkb_rows - 1) // nkb_rows
        buf = torch.zeros((nkb + 1) * n, dtype=torch.float32, device=dev)

        def run(mode):
            _lib.check("jattn_probe_dq_accumulation",
                       lib.jattn_probe_dq_accumulation(mode, pairs, L, D, nkb, buf.data_ptr(), buf.numel() * 4, sp))

        for mode, name in ((0, "atomic"), (1, "partial_store"), (2, "partial_reduce")):
            times = []
            for rep in range(6):
                if mode == 0:
                    buf[:n].zero_()
                a, b = new_event(), new_event()
                a.record(stream)
                run(mode)
                b.record(stream)
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
            ent = {"mode": name, "key_block_rows": nkb_rows, "key_blocks": nkb, "ms": round(min(times), 5)}
            if mode == 0:
                ok = bool(torch.all(buf[:n] == float(nkb)).item())
                ent.update({"g_atomics_per_s": round(nkb * n / (min(times) * 1e-3) / 1e9, 1), "sums_exact": ok})
            else:
                moved = (nkb * n if mode == 1 else (nkb + 1) * n) * 4
                ent["gbs"] = round(moved / (min(times) * 1e-3) / 1e9, 1)
            res["modes"].append(ent)
        del buf
    print(json.dumps(res), flush=True)


def probe_tile(torch):
    """The probes of jattn_diag.h that time the dk/dv tile's dependency structure (which operands come from
    LDS), the LDS read rates and the MFMA / VALU issue rates, on the shader clock. Prints one JSON line."""
    from diffusion_transformer_joint_amd import _lib
    lib = _lib.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sp = torch.cuda.current_stream().cuda_stream
    modes = ("registers", "lds", "lds_barrier", "rows_stats", "transposed", "stats", "rows", "pipelined")
    res = {"what": "dk/dv tile dependency structure at D = 64 (32 MFMAs of 32x32x16 per wave and tile) and LDS "
                   "read rates; shader-clock cycles from s_memtime", "compute_units": cus, "tile": [], "lds_read": []}
    iters = 2000
    for wps in (1, 2):
        blocks = cus * wps
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
        cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda:0")
        for mode, name in enumerate(modes):
            for _ in range(2):  # (the first launch warms the clocks)
                _lib.check("jattn_probe_tile", lib.jattn_probe_tile(mode, blocks, iters, ctypes.c_float(1e-3),
                                                                    out.data_ptr(), cyc.data_ptr(), sp))
            torch.cuda.synchronize()
            c = cyc.double() / iters
            res["tile"].append({"mode": name, "waves_per_simd": wps, "cycles_per_tile_mean": round(c.mean().item(), 1),
                                "min": round(c.min().item(), 1), "max": round(c.max().item(), 1),
                                "mfma_busy": round(1024.0 * wps / c.mean().item(), 3)})
    for wgs in (1, 2):
        blocks = cus * wgs
        cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda:0")
        for mode, (name, width) in enumerate((("b128", 16), ("b128_broadcast", 16), ("b64_transposed", 8))):
            for _ in range(2):
                _lib.check("jattn_probe_lds_read", lib.jattn_probe_lds_read(mode, blocks, 4000, cyc.data_ptr(), sp))
            torch.cuda.synchronize()
            c = cyc.double().mean().item()
            res["lds_read"].append({"read": name, "waves_per_cu": 4 * wgs,
                                    "bytes_per_cu_per_cycle": round(8 * 4000 * 64 * width * 4 * wgs / c, 1),
                                    "cycles_per_wave_instruction": round(c / (8 * 4000), 2)})
    # Issue rates (jattn_probe_issue): one workgroup of 8 waves per compute unit, two waves per SIMD.
    # Per SIMD, the slower of its two waves over the 8 * iters steps is the SIMD's cycles per step of both.
    res["issue"] = []
    iters = 4000
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda:0")
    cyc = torch.zeros(cus * 8, dtype=torch.int64, device="cuda:0")
    steps = (("mfma", "1 MFMA in each wave"), ("fma", "16 FMAs in each wave"), ("exp", "8 exp2 in each wave"),
             ("mixed_fma", "1 MFMA + 16 FMAs in each wave"), ("mixed_exp", "1 MFMA + 8 exp2 in each wave"),
             ("split_fma", "1 MFMA in one wave, 16 FMAs in the other"),
             ("split_exp", "1 MFMA in one wave, 8 exp2 in the other"))
    for mode, (name, step) in enumerate(steps):
        for _ in range(2):
            _lib.check("jattn_probe_issue", lib.jattn_probe_issue(mode, cus, iters, ctypes.c_float(1e-3),
                                                                  out.data_ptr(), cyc.data_ptr(), sp))
        torch.cuda.synchronize()
        c = cyc.view(cus, 2, 4).double() / (8 * iters)  # [cu, wave pair slot, simd]
        simd = torch.maximum(c[:, 0, :], c[:, 1, :])
        res["issue"].append({"mode": name, "step_per_wave": step, "simd_cycles_per_step": round(simd.mean().item(), 1),
                             "waves_0_3_cycles_per_step": round(c[:, 0, :].mean().item(), 1),
                             "waves_4_7_cycles_per_step": round(c[:, 1, :].mean().item(), 1)})
    # The forward tile's schedules (jattn_probe_pingpong): 16 MFMAs per wave and step, two waves per SIMD.
    res["pingpong"] = []
    iters = 2000
    for mode, name in enumerate(("free", "barrier_per_step", "phased")):
        for lds in (0, 1):
            for _ in range(2):
                _lib.check("jattn_probe_pingpong", lib.jattn_probe_pingpong(mode, lds, cus, iters, ctypes.c_float(1e-3),
                                                                            out.data_ptr(), cyc.data_ptr(), sp))
            torch.cuda.synchronize()
            c = cyc.double() / iters
            res["pingpong"].append({"schedule": name, "operands": "lds" if lds else "registers",
                                    "cycles_per_step_mean": round(c.mean().item(), 1),
                                    "cycles_per_step_max": round(c.max().item(), 1),
                                    "mfma_busy_mean": round(1024.0 / c.mean().item(), 3),
                                    "mfma_busy_slowest_wave": round(1024.0 / c.max().item(), 3)})
    print(json.dumps(res), flush=True)


def run_busy_probes(torch):
    """The saturating probes of jattn_diag.h on every SIMD (8 waves each): MFMA only, then FMA only."""
    from diffusion_transformer_joint_amd import _lib
    lib = _lib.load()
    blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    sp = torch.cuda.current_stream().cuda_stream
    for which, iters in ((0, 128), (1, 1024)):
        _lib.check("jattn_probe_saturate", lib.jattn_probe_saturate(which, blocks, iters, ctypes.c_float(1.0),
                                                                    out.data_ptr(), sp))
    torch.cuda.synchronize()


def time_cold_steps(torch, stream, fwd, bwd, new_event, K):
    """Per-step times with a 512 MiB write (outside the measured span) before each step, so that no
    operand is left in the L2 or the Infinity Cache from the previous step."""
    junk = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=stream.device)
    evs = [[new_event() for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        junk.fill_(float(i))
        evs[i][0].record(stream)
        fwd()
        evs[i][1].record(stream)
        bwd()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    spread = lambda xs: {"median": round(sorted(xs)[len(xs) // 2], 5), "min": round(min(xs), 5)}
    res = {"fwd": spread([e[0].elapsed_time(e[1]) for e in evs]), "bwd": spread([e[1].elapsed_time(e[2]) for e in evs]),
           "fwd+bwd": spread([e[0].elapsed_time(e[2]) for e in evs]), "steps": K,
           "note": "512 MiB written before each step, outside the measured span"}
    del junk
    return res


def breakdown_pass(fwd, bwd, stages, nfs, KB, stream, new_event, handle):
    """Per-stage average durations over KB steps with every stage event recorded (outside the timed
    region), and the forward's share of the step."""
    import torch
    ev0 = [new_event() for _ in range(KB)]
    evb = [[new_event() for _ in stages] for _ in range(KB)]
    fh = [handle(evb[i][:nfs]) for i in range(KB)]
    bhh = [handle(evb[i][nfs:]) for i in range(KB)]
    torch.cuda.synchronize()
    for i in range(KB):
        ev0[i].record(stream)
        fwd(fh[i][1])
        bwd(bhh[i][1])
    torch.cuda.synchronize()
    kern_ms = {}
    for j, name in enumerate(stages):
        kern_ms[name] = sum((ev0[i] if j == 0 else evb[i][j - 1]).elapsed_time(evb[i][j]) for i in range(KB)) / KB
    ms_fwd = sum(ev0[i].elapsed_time(evb[i][nfs - 1]) for i in range(KB)) / KB
    ms_bwd = sum(evb[i][nfs - 1].elapsed_time(evb[i][-1]) for i in range(KB)) / KB
    return kern_ms, ms_fwd, ms_bwd


def timed_region(fwd, bwd, j, nfs, K, stream, new_event, handle):
    """K whole steps between two events. The library's own stage events bracket stage j (of the
    forward's nfs stages followed by the backward's) in every step, so that stage's average launch
    duration is measured live, on the stream the kernels run on. Only the two events around stage j
    are recorded (the entries for the earlier stages are NULL): each recorded event costs the stream
    a few microseconds."""
    import torch
    jb = j - nfs
    n = (j if jb < 0 else jb) + 1  # stage events handed to the pass that runs stage j
    ev = [[new_event() if s >= n - 2 else None for s in range(n)] for _ in range(K)]
    pre = [new_event() for _ in range(K)] if n == 1 else None  # stage j is that pass's first
    hs = [handle(ev[i]) for i in range(K)]
    start, end = new_event(), new_event()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        if jb < 0:
            if pre is not None:
                pre[i].record(stream)
            fwd(hs[i][1], n)
            bwd()
        else:
            fwd()
            if pre is not None:
                pre[i].record(stream)
            bwd(hs[i][1], n)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    dom_ms = sum((pre[i] if pre is not None else ev[i][-2]).elapsed_time(ev[i][-1]) for i in range(K)) / K
    return ms_step, dom_ms


ADALN_METRIC = "adaLN+QKV projection fwd+bwd TFLOP/s (both streams) bf16; % of bf16 MFMA peak"


def bench_adaln(args, torch):
    """The adaLN-modulated QKV projection of one layer, forward + backward over both streams."""
    from diffusion_transformer_joint_amd import _lib
    from diffusion_transformer_joint_amd.inputs import ADALN_WORKLOADS, adaln_flops, make_workload_adaln_inputs

    if args.workload not in ADALN_WORKLOADS:
        args.workload = "mmdit512"
    w = ADALN_WORKLOADS[args.workload]
    B, C = w.B, w.C
    inp = make_workload_adaln_inputs(args.workload, seed=0)
    dev = torch.device("cuda:0")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in ("x", "mod", "w", "bias", "dq", "dk", "dv")}
    lib = _lib.load()
    fws_bytes = int(lib.jattn_adaln_qkv_fwd_workspace_bytes(B, w.n_img, w.n_txt, C))
    ws_bytes = int(lib.jattn_adaln_qkv_bwd_workspace_bytes(B, w.n_img, w.n_txt, C))
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ns = (w.n_img, w.n_txt)
    q, k, v, dx = ([torch.empty(B, n, C, dtype=torch.bfloat16, device=dev) for n in ns] for _ in range(4))
    dmod = [torch.empty(B, 2, C, dtype=torch.float32, device=dev) for _ in ns]
    dw = [torch.empty(3 * C, C, dtype=torch.float32, device=dev) for _ in ns]
    db = [torch.empty(3 * C, dtype=torch.float32, device=dev) for _ in ns]
    pp = lambda t: _lib.PtrPair(t[0].data_ptr(), t[1].data_ptr())
    keep = {n: pp(t) for n, t in (("x", d["x"]), ("mod", d["mod"]), ("w", d["w"]), ("bias", d["bias"]), ("q", q),
                                  ("k", k), ("v", v), ("dq", d["dq"]), ("dk", d["dk"]), ("dv", d["dv"]), ("dx", dx),
                                  ("dmod", dmod), ("dw", dw), ("db", db))}
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    nfs, nbs = len(_lib.ADALN_FWD_STAGES), len(_lib.ADALN_BWD_STAGES)

    def fwd(events=None, n=nfs):
        _lib.check("jattn_adaln_qkv_fwd", lib.jattn_adaln_qkv_fwd(
            keep["x"].arg, keep["mod"].arg, keep["w"].arg, keep["bias"].arg, B, w.n_img, w.n_txt, C,
            ctypes.c_float(inp["eps"]), keep["q"].arg, keep["k"].arg, keep["v"].arg, fws.data_ptr(), fws_bytes,
            events, 0 if events is None else n, sp))

    def bwd(events=None, n=nbs):
        _lib.check("jattn_adaln_qkv_bwd", lib.jattn_adaln_qkv_bwd(
            keep["x"].arg, keep["mod"].arg, keep["w"].arg, keep["dq"].arg, keep["dk"].arg, keep["dv"].arg, B,
            w.n_img, w.n_txt, C, keep["dx"].arg, keep["dmod"].arg, keep["dw"].arg, keep["db"].arg, fws.data_ptr(),
            fws_bytes, ws.data_ptr(), ws_bytes, events, 0 if events is None else n, sp))

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def handle(evs):
        arr = (ctypes.c_void_p * len(evs))(*[None if e is None else e.cuda_event for e in evs])
        return arr, ctypes.cast(arr, ctypes.c_void_p)

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    pre = preroll(torch, stream, lambda: (fwd(), bwd()), new_event)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    K = args.steps
    targs = {"qkv_gemm_kernel": "256, 256, 2, 8", "dh_gemm_kernel": "256, 256, 2, false, 8",
             "dw_gemm_kernel": "256, 256, 2, 8"}
    label = lambda n: f"{n}<{targs[n]}>" if n in targs else n
    stages = [label(n) + " (fwd)" if n == "modulate_kernel" else label(n) for n in _lib.ADALN_FWD_STAGES]
    stages += [label(n) for n in _lib.ADALN_BWD_STAGES]
    kern_ms, ms_fwd, ms_bwd = breakdown_pass(fwd, bwd, stages, nfs, min(K, 50), stream, new_event, handle)
    gemms = [label(n) for n in ("qkv_gemm_kernel", "dh_gemm_kernel", "dw_gemm_kernel")]
    dom = max(gemms, key=lambda n: kern_ms[n])
    ms_step, dom_ms = timed_region(fwd, bwd, stages.index(dom), nfs, K, stream, new_event, handle)

    fl = adaln_flops(B, w.n_img, w.n_txt, C)
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12
    achieved = fl["fwd"] / (dom_ms * 1e-3) / 1e12  # each GEMM is 2 T C 3C FLOPs per launch
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(args.workload, dom, "adaln"), "flop_per_launch": fl["fwd"],
                "avg_launch_ms": round(dom_ms, 5), "avg_launch_ms_source": "timed region"}

    unfused = time_adaln_unfused(torch, d, inp, stream, K, args.warmup)
    cpu = None if args.no_cpu_baseline else cpu_baseline_adaln(inp, args.cpu_seconds)
    res = {
        "metric": ADALN_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "variant": "adaln", "B": B, "n_img": w.n_img, "n_txt": w.n_txt,
                   "C": C, "global_batch": B, "parallelism": "single-gpu"},
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(ms_fwd, 5), "bwd_ms": round(ms_bwd, 5), "preroll": pre,
        "fwd_bwd_source": "breakdown pass (both from the same pass)",
        "gflop_per_step": round(fl["total"] / 1e9, 3),
        "kernel_ms": {k: round(v, 5) for k, v in kern_ms.items()},
        "roofline": roofline, "cpu_baseline": cpu,
        "torch_unfused": {"ms_per_step": round(unfused, 5), "speedup": round(unfused / ms_step, 4),
                          "what": "torch: layer_norm, * (1 + scale) + shift, linear, split into q, k, v, and "
                                  "autograd backward with the same upstream gradients, both streams, bf16"},
    }
    print(json.dumps(res), flush=True)


MLP_METRIC = "MLP block (fc, adaLN, SwiGLU, residual) fwd+bwd TFLOP/s (both streams) bf16; % of bf16 MFMA peak"


def bench_mlp(args, torch):
    """The MLP block of one layer, forward + backward over both streams."""
    from diffusion_transformer_joint_amd import _lib
    from diffusion_transformer_joint_amd.inputs import MLP_WORKLOADS, make_workload_mlp_inputs, mlp_flops

    if args.workload not in MLP_WORKLOADS:
        args.workload = "mmdit512"
    w = MLP_WORKLOADS[args.workload]
    B, C, Fh = w.B, w.C, w.F
    inp = make_workload_mlp_inputs(args.workload, seed=0)
    dev = torch.device("cuda:0")
    keys = ("o", "x", "mod", "wfc", "bfc", "w12", "b12", "w2", "b2", "dout")
    d = {k: tuple(t.to(dev).contiguous() for t in inp[k]) for k in keys}
    lib = _lib.load()
    dims = (B, w.n_img, w.n_txt, C, Fh)
    fws_bytes, ws_bytes = int(lib.jattn_mlp_fwd_workspace_bytes(*dims)), int(lib.jattn_mlp_bwd_workspace_bytes(*dims))
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ns = (w.n_img, w.n_txt)
    out, do = ([torch.empty(B, n, C, dtype=torch.bfloat16, device=dev) for n in ns] for _ in range(2))
    f32 = lambda *shape: [torch.empty(*shape, dtype=torch.float32, device=dev) for _ in ns]
    g = dict(dmod=f32(B, 2, C), dwfc=f32(C, C), dbfc=f32(C), dw12=f32(2 * Fh, C), db12=f32(2 * Fh), dw2=f32(C, Fh),
             db2=f32(C))
    pp = lambda t: _lib.PtrPair(t[0].data_ptr(), t[1].data_ptr())
    keep = {k: pp(d[k]) for k in keys}
    keep.update(out=pp(out), do=pp(do), **{k: pp(v) for k, v in g.items()})
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    nfs, nbs = len(_lib.MLP_FWD_STAGES), len(_lib.MLP_BWD_STAGES)
    a = lambda *names: [keep[n].arg for n in names]

    def fwd(events=None, n=nfs):
        _lib.check("jattn_mlp_fwd", lib.jattn_mlp_fwd(*a("o", "x", "mod", "wfc", "bfc", "w12", "b12", "w2", "b2"), *dims,
                                                      ctypes.c_float(inp["eps"]), keep["out"].arg, fws.data_ptr(),
                                                      fws_bytes, events, 0 if events is None else n, sp))

    def bwd(events=None, n=nbs):
        _lib.check("jattn_mlp_bwd", lib.jattn_mlp_bwd(*a("o", "mod", "wfc", "w12", "w2", "dout"), *dims,
                                                      *a("do", "dmod", "dwfc", "dbfc", "dw12", "db12", "dw2", "db2"),
                                                      fws.data_ptr(), fws_bytes, ws.data_ptr(), ws_bytes, events,
                                                      0 if events is None else n, sp))

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def handle(evs):
        arr = (ctypes.c_void_p * len(evs))(*[None if e is None else e.cuda_event for e in evs])
        return arr, ctypes.cast(arr, ctypes.c_void_p)

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    pre = preroll(torch, stream, lambda: (fwd(), bwd()), new_event)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    K = args.steps
    # stage labels: kernel instantiations (the forward's fc and down projection and the backward's do
    # GEMM are the bf16-output GEMM; du the fp32-output one; d(hid) that one with the SwiGLU epilogue)
    lab = {"fc_gemm": "qkv_gemm_kernel<256, 256, 2, 8> (fc)", "modulate_kernel": "modulate_kernel",
           "swiglu_gemm_kernel": "swiglu_gemm_kernel<256, 256, 2, 8>",
           "down_gemm": "qkv_gemm_kernel<256, 256, 2, 8> (down)", "transpose_w_kernel": "transpose_w_kernel",
           "dhid_gemm": "dh_gemm_kernel<256, 256, 2, true, 8> (d hid)",
           "dw2_gemm": "dw_gemm_kernel<256, 256, 2, 8> (dW2)", "du_gemm": "dh_gemm_kernel<256, 256, 2, false, 8> (du)",
           "dw12_gemm": "dw_gemm_kernel<256, 256, 2, 8> (dW12)", "rows_bwd_kernel": "rows_bwd_kernel",
           "do_gemm": "qkv_gemm_kernel<256, 256, 2, 8> (do)", "dwfc_gemm": "dw_gemm_kernel<256, 256, 2, 8> (dWfc)",
           "reductions": "reductions"}
    stages = [lab[n] for n in _lib.MLP_FWD_STAGES] + [lab[n] for n in _lib.MLP_BWD_STAGES]
    kern_ms, ms_fwd, ms_bwd = breakdown_pass(fwd, bwd, stages, nfs, min(K, 50), stream, new_event, handle)
    T = B * (w.n_img + w.n_txt)
    # GEMM FLOPs per launch (2 T x output x contraction); the dominant one is the largest by time
    per_launch = {lab["fc_gemm"]: 2.0 * T * C * C, lab["swiglu_gemm_kernel"]: 2.0 * T * 2 * Fh * C,
                  lab["down_gemm"]: 2.0 * T * C * Fh, lab["dhid_gemm"]: 2.0 * T * Fh * C,
                  lab["dw2_gemm"]: 2.0 * T * C * Fh, lab["du_gemm"]: 2.0 * T * C * 2 * Fh,
                  lab["dw12_gemm"]: 2.0 * T * 2 * Fh * C, lab["do_gemm"]: 2.0 * T * C * C, lab["dwfc_gemm"]: 2.0 * T * C * C}
    dom = max(per_launch, key=lambda n: kern_ms[n])
    ms_step, dom_ms = timed_region(fwd, bwd, stages.index(dom), nfs, K, stream, new_event, handle)

    fl = mlp_flops(B, w.n_img, w.n_txt, C, Fh)
    tflops = fl["total"] / (ms_step * 1e-3) / 1e12
    achieved = per_launch[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(args.workload, dom, "mlp"), "flop_per_launch": per_launch[dom],
                "avg_launch_ms": round(dom_ms, 5), "avg_launch_ms_source": "timed region"}

    unfused = time_mlp_unfused(torch, d, inp, stream, K, args.warmup)
    cpu = None if args.no_cpu_baseline else cpu_baseline_mlp(inp, args.cpu_seconds)
    res = {
        "metric": MLP_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "variant": "mlp", "B": B, "n_img": w.n_img, "n_txt": w.n_txt, "C": C,
                   "F": Fh, "global_batch": B, "parallelism": "single-gpu"},
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(ms_fwd, 5), "bwd_ms": round(ms_bwd, 5), "preroll": pre,
        "fwd_bwd_source": "breakdown pass (both from the same pass)",
        "gflop_per_step": round(fl["total"] / 1e9, 3),
        "kernel_ms": {k: round(v, 5) for k, v in kern_ms.items()},
        "roofline": roofline, "cpu_baseline": cpu,
        "torch_unfused": {"ms_per_step": round(unfused, 5), "speedup": round(unfused / ms_step, 4),
                          "what": "torch: linear, layer_norm, * (1 + scale) + shift, linear, silu * gate, linear, "
                                  "+ residual, and autograd backward, both streams, bf16"},
    }
    print(json.dumps(res), flush=True)


def time_mlp_unfused(torch, d, inp, stream, K, warmup):
    """The same block step in plain torch ops (separate kernels, hipBLASLt GEMMs), forward + autograd
    backward."""
    import torch.nn.functional as F
    C = inp["C"]
    leaf = {k: tuple(t.clone().requires_grad_(True) for t in d[k]) for k in ("o", "x", "mod")}
    par = {k: [t.detach().clone().to(torch.bfloat16).requires_grad_(True) for t in d[k]]
           for k in ("wfc", "bfc", "w12", "b12", "w2", "b2")}

    def step():
        outs, grads = [], []
        for s in range(2):
            m = leaf["mod"][s].to(torch.bfloat16)
            z = F.linear(leaf["o"][s], par["wfc"][s], par["bfc"][s])
            u = F.layer_norm(z, (C,), eps=inp["eps"]) * (1 + m[:, 1:2]) + m[:, 0:1]
            a, g = F.linear(u, par["w12"][s], par["b12"][s]).chunk(2, dim=-1)
            outs.append(leaf["x"][s] + F.linear(F.silu(a) * g, par["w2"][s], par["b2"][s]))
            grads.append(d["dout"][s])
        torch.autograd.backward(outs, grads)

    return time_steps(torch, stream, step, K, warmup)


def cpu_baseline_mlp(inp, seconds):
    """The fp64 oracle (mlp_fwd_bwd) on whole samples of the image stream, as many as fit the time budget
    (at least one), in TFLOP/s of the GEMM FLOPs it covered."""
    from oracle import mlp_fwd_bwd
    f64 = lambda t: t.double().numpy()
    B, C, Fh, n = inp["B"], inp["C"], inp["F"], inp["n_img"]
    t0 = time.perf_counter()
    done = 0
    while done < B and (done == 0 or time.perf_counter() - t0 < seconds):
        sl = slice(done, done + 1)
        t = lambda k: f64(inp[k][0][sl])
        wt = lambda k: f64(inp[k][0])
        mlp_fwd_bwd(t("o"), t("x"), t("mod"), wt("wfc"), wt("bfc"), wt("w12"), wt("b12"), wt("w2"), wt("b2"), inp["eps"],
                    t("dout"))
        done += 1
    sec = time.perf_counter() - t0
    flop = 3 * 2.0 * done * n * (C * C + 3 * C * Fh)
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    return {"value": round(flop / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle (mlp_fwd_bwd) fwd+bwd on the first {done} of {B} samples of the image "
                      f"stream ({n} tokens each) of the same seed-0 inputs, {sec:.1f} s wall; BLAS threads = cores",
            "seconds": round(sec, 2), "samples": done}


def time_adaln_unfused(torch, d, inp, stream, K, warmup):
    """The same layer step in plain torch ops (LayerNorm, modulation and Linear as separate kernels,
    hipBLASLt GEMMs), forward + autograd backward, timed the same way."""
    import torch.nn.functional as F
    C = inp["C"]
    leaf = {k: tuple(t.clone().requires_grad_(True) for t in d[k]) for k in ("x", "mod", "w", "bias")}
    wb = [t.detach().clone().to(torch.bfloat16).requires_grad_(True) for t in leaf["w"]]
    bb = [t.detach().clone().to(torch.bfloat16).requires_grad_(True) for t in leaf["bias"]]

    def step():
        outs, grads = [], []
        for s in range(2):
            x = leaf["x"][s]
            m = leaf["mod"][s].to(torch.bfloat16)
            h = F.layer_norm(x, (C,), eps=inp["eps"]) * (1 + m[:, 1:2]) + m[:, 0:1]
            y = F.linear(h, wb[s], bb[s])
            outs += list(y.split(C, dim=-1))
            grads += [d[n][s] for n in ("dq", "dk", "dv")]
        torch.autograd.backward(outs, grads)

    return time_steps(torch, stream, step, K, warmup)


def cpu_baseline_adaln(inp, seconds):
    """The fp64 oracle (adaln_qkv_fwd_bwd) on whole samples of the image stream, as many as fit the time
    budget (at least one), in TFLOP/s of the GEMM FLOPs it covered."""
    import numpy as np
    from oracle import adaln_qkv_fwd_bwd
    f64 = lambda t: t.double().numpy()
    B, C, n = inp["B"], inp["C"], inp["n_img"]
    t0 = time.perf_counter()
    done = 0
    while done < B and (done == 0 or time.perf_counter() - t0 < seconds):
        sl = slice(done, done + 1)
        g = lambda key: f64(inp[key][0][sl]).reshape(1, n, 1, C)
        adaln_qkv_fwd_bwd(f64(inp["x"][0][sl]), f64(inp["mod"][0][sl]), f64(inp["w"][0]), f64(inp["bias"][0]), 1,
                          inp["eps"], g("dq"), g("dk"), g("dv"))
        done += 1
    sec = time.perf_counter() - t0
    flop = 3 * 2.0 * done * n * C * 3 * C
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    return {"value": round(flop / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle (adaln_qkv_fwd_bwd) fwd+bwd on the first {done} of {B} samples of the "
                      f"image stream ({n} tokens each) of the same seed-0 inputs, {sec:.1f} s wall; BLAS threads "
                      "= cores", "seconds": round(sec, 2), "samples": done}


def time_concat_split(lib, _lib, torch, q, k, v, dout, gains, vl, B, L, H, D, inp, stream, K, warmup):
    """The step the two-stream entry points replace, timed the same way: concatenate the image and text
    parts of q, k, v (and dout), run the joint forward and backward, split out, dq, dk and dv back
    into per-stream tensors. The joint kernels take one gain pair, so the image stream's gains stand
    in for both (the kernel work is the same)."""
    n_img = q[0].shape[1]
    g0 = gains[0].contiguous()
    vlp = None if vl is None else vl.data_ptr()
    lse = torch.empty(B, H, L, dtype=torch.float32, device=q[0].device)
    fws_bytes = int(lib.jattn_fwd_workspace_bytes(B, L, H, D))
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=q[0].device)
    ws_bytes = int(lib.jattn_bwd_workspace_bytes(B, L, H, D))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q[0].device)
    scale, eps = ctypes.c_float(inp["scale"]), ctypes.c_float(inp["eps"])
    sp = stream.cuda_stream

    def step():
        qj, kj, vj = (torch.cat(t, dim=1) for t in (q, k, v))
        out = torch.empty_like(qj)
        _lib.check("jattn_fwd", lib.jattn_fwd(qj.data_ptr(), kj.data_ptr(), vj.data_ptr(), g0.data_ptr(), vlp, B, L,
                                              H, D, scale, eps, out.data_ptr(), lse.data_ptr(), fws.data_ptr(),
                                              fws_bytes, sp))
        outs = (out[:, :n_img].contiguous(), out[:, n_img:].contiguous())
        doj = torch.cat(dout, dim=1)
        dq, dk, dv = torch.empty_like(qj), torch.empty_like(kj), torch.empty_like(vj)
        dg = torch.empty(2, D, dtype=torch.float32, device=qj.device)
        _lib.check("jattn_bwd", lib.jattn_bwd(qj.data_ptr(), kj.data_ptr(), vj.data_ptr(), g0.data_ptr(), vlp,
                                              out.data_ptr(), lse.data_ptr(), doj.data_ptr(), B, L, H, D, scale, eps,
                                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dg.data_ptr(),
                                              ws.data_ptr(), ws_bytes, fws.data_ptr(), sp))
        return outs, [(t[:, :n_img].contiguous(), t[:, n_img:].contiguous()) for t in (dq, dk, dv)]

    for _ in range(min(warmup, 20)):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    return {"ms_per_step": round(ms, 5),
            "what": "torch.cat of the q, k, v and dout parts + jattn_fwd + jattn_bwd + .contiguous() splits of "
                    "out, dq, dk, dv (same workload and stream)"}


def time_steps(torch, stream, step, K, warmup):
    """Average ms of `step` over K calls after a short warm-up, by events around all of them."""
    for _ in range(min(warmup, 20)):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def window_flops(B, L, H, D, valid_len, window):
    """Algorithmic FLOPs under a local window: 4*D per (query, key) pair the window and the key padding
    allow, backward 2.5x."""
    import numpy as np
    left, right = window
    i = np.arange(L)
    lo = np.zeros(L, dtype=np.int64) if left < 0 else np.maximum(0, i - left)
    pairs = 0
    for b in range(B):
        n = L if valid_len is None else max(0, min(L, int(valid_len[b])))
        hi = np.full(L, n, dtype=np.int64) if right < 0 else np.minimum(n, i + right + 1)
        pairs += int(np.maximum(0, hi - lo).sum())
    fwd = 4.0 * H * D * pairs
    return dict(fwd=fwd, bwd=2.5 * fwd, total=3.5 * fwd)


def time_padded(lib, _lib, torch, inp, gains, B, L, H, D, stream, K, warmup):
    """The same sequences padded to the longest one (L rows each, zeros after each sequence's end),
    run through the joint entry points with valid_len = the lengths: what a packed batch replaces."""
    dev = gains.device
    lengths, cu = inp["lengths"], inp["cu_seqlens"].tolist()
    pad = lambda t: torch.stack([torch.cat([t[cu[b]:cu[b + 1]], torch.zeros(L - n, H, D, dtype=t.dtype)])
                                 for b, n in enumerate(lengths)]).to(dev)
    q, k, v, dout = (pad(inp[n]) for n in ("q", "k", "v", "dout"))
    vl = torch.tensor(lengths, dtype=torch.int32, device=dev)
    out, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(B, H, L, dtype=torch.float32, device=dev)
    dg = torch.empty(2, D, dtype=torch.float32, device=dev)
    fws_bytes, ws_bytes = int(lib.jattn_fwd_workspace_bytes(B, L, H, D)), int(lib.jattn_bwd_workspace_bytes(B, L, H, D))
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scale, eps = ctypes.c_float(inp["scale"]), ctypes.c_float(inp["eps"])
    sp = stream.cuda_stream

    def step():
        _lib.check("jattn_fwd", lib.jattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), vl.data_ptr(),
                                              B, L, H, D, scale, eps, out.data_ptr(), lse.data_ptr(), fws.data_ptr(),
                                              fws_bytes, sp))
        _lib.check("jattn_bwd", lib.jattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), vl.data_ptr(),
                                              out.data_ptr(), lse.data_ptr(), dout.data_ptr(), B, L, H, D, scale, eps,
                                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dg.data_ptr(), ws.data_ptr(),
                                              ws_bytes, fws.data_ptr(), sp))

    for _ in range(min(warmup, 20)):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return {"ms_per_step": round(a.elapsed_time(b) / K, 5),
            "what": f"the same sequences padded to L = {L} (B = {B}), jattn_fwd + jattn_bwd with valid_len = the "
                    "lengths (padded query rows are computed, padded keys masked)"}


def cpu_baseline(inp, seconds):
    """The fp64 oracle (as is) on the first (batch, head) pairs of the same inputs, time-bounded."""
    import numpy as np
    import torch

    from oracle import attention_fwd_bwd, streams_fwd_bwd, varlen_fwd_bwd

    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    w = inp["workload"]
    if "cu_seqlens" in inp:
        return cpu_baseline_varlen(inp, seconds, threads, varlen_fwd_bwd)
    B, L, H, D = w.B, w.L, w.H, w.D
    f = lambda t: tuple(f(x) for x in t) if isinstance(t, tuple) else t.to(torch.float64).numpy()
    q, k, v, do = (f(inp[n]) for n in ("q", "k", "v", "dout"))
    g = inp["gains"].double().numpy()
    run = streams_fwd_bwd if isinstance(q, tuple) else attention_fwd_bwd
    vl = None if inp["valid_len"] is None else inp["valid_len"].tolist()
    pairs = [(b, h) for b in range(B) for h in range(H)]
    done, flop = 0, 0.0
    t0 = time.perf_counter()
    chunk = 4
    while done < len(pairs) and time.perf_counter() - t0 < seconds:
        sel = pairs[done:done + chunk]
        run(q, k, v, g, do, vl, inp["scale"], inp["eps"], pairs=sel)
        for b, _ in sel:
            n = L if vl is None else max(0, min(L, vl[b]))
            flop += 3.5 * 4.0 * L * n * D
        done += len(sel)
    dt = time.perf_counter() - t0
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle ({run.__name__}) fwd+bwd on the first {done} of {len(pairs)} (batch, head) pairs of "
                      f"the same seed-0 inputs, {dt:.1f} s wall; BLAS threads = cores, elementwise steps "
                      f"single-threaded",
            "seconds": round(dt, 2), "pairs": done}


def cpu_baseline_varlen(inp, seconds, threads, varlen_fwd_bwd):
    """The fp64 variable-length oracle on the first sequences of the same packed inputs, time-bounded."""
    import torch
    w = inp["workload"]
    f = lambda t: t.to(torch.float64).numpy()
    q, k, v, do = (f(inp[n]) for n in ("q", "k", "v", "dout"))
    g = inp["gains"].double().numpy()
    cu = inp["cu_seqlens"].tolist()
    done, flop = 0, 0.0
    t0 = time.perf_counter()
    while done < w.B and time.perf_counter() - t0 < seconds:
        varlen_fwd_bwd(q, k, v, g, do, cu, inp["scale"], inp["eps"], seqs=[done])
        n = cu[done + 1] - cu[done]
        flop += 3.5 * 4.0 * w.H * n * n * w.D
        done += 1
    dt = time.perf_counter() - t0
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle (varlen_fwd_bwd) fwd+bwd on the first {done} of {w.B} sequences of the "
                      f"same seed-0 packed inputs, {dt:.1f} s wall; BLAS threads = cores",
            "seconds": round(dt, 2), "sequences": done}


if __name__ == "__main__":
    main()
