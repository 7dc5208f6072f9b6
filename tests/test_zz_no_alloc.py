"""The allocation-free forward entry point (jattn_fwd_noalloc) through the C ABI: its outputs against
those of jattn_fwd with a caller workspace, bit for bit (the same kernels), on two calls in a row
(the second with a smaller input, so the scratch array holds the first call's rows), followed by the
backward from its outputs. (Its host-side refusals are in test_abi.py.)"""
import ctypes

import numpy as np
import pytest
import torch

from diffusion_transformer_joint_amd import _lib
from diffusion_transformer_joint_amd.inputs import make_shape_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_both(lib, inp):
    dev = torch.device("cuda:0")
    q, k, v, g, dout = (inp[n].to(dev).contiguous() for n in ("q", "k", "v", "gains", "dout"))
    vl = None if inp["valid_len"] is None else inp["valid_len"].to(dev)
    vlp = None if vl is None else vl.data_ptr()
    B, L, H, D = q.shape
    sp = torch.cuda.current_stream().cuda_stream
    scale, eps = ctypes.c_float(inp["scale"]), ctypes.c_float(inp["eps"])
    out_a, out_b = torch.empty_like(q), torch.empty_like(q)
    lse_a, lse_b = (torch.empty(B * H * L, dtype=torch.float32, device=dev) for _ in range(2))
    fb = int(lib.jattn_fwd_workspace_bytes(B, L, H, D))
    fws = torch.empty(fb, dtype=torch.uint8, device=dev)
    _lib.check("jattn_fwd", lib.jattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), vlp, B, L, H, D,
                                          scale, eps, out_a.data_ptr(), lse_a.data_ptr(), fws.data_ptr(), fb, sp))
    _lib.check("jattn_fwd_noalloc", lib.jattn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), vlp,
                                                          B, L, H, D, scale, eps, out_b.data_ptr(), lse_b.data_ptr(),
                                                          sp))
    # the backward of the allocation-free forward: jattn_bwd normalising the keys itself
    bb = int(lib.jattn_bwd_workspace_bytes(B, L, H, D))
    ws = torch.empty(bb, dtype=torch.uint8, device=dev)
    grads = [torch.empty_like(q) for _ in range(3)] + [torch.empty(2, D, dtype=torch.float32, device=dev)]
    _lib.check("jattn_bwd", lib.jattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), vlp, out_b.data_ptr(),
                                          lse_b.data_ptr(), dout.data_ptr(), B, L, H, D, scale, eps,
                                          grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                          grads[3].data_ptr(), ws.data_ptr(), bb, None, sp))
    ref = [torch.empty_like(t) for t in grads]
    _lib.check("jattn_bwd", lib.jattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), vlp, out_a.data_ptr(),
                                          lse_a.data_ptr(), dout.data_ptr(), B, L, H, D, scale, eps,
                                          ref[0].data_ptr(), ref[1].data_ptr(), ref[2].data_ptr(), ref[3].data_ptr(),
                                          ws.data_ptr(), bb, fws.data_ptr(), sp))
    torch.cuda.synchronize()
    return (out_a, lse_a, ref), (out_b, lse_b, grads)


def test_noalloc_forward_matches_workspace_forward():
    lib = _lib.load()
    # first call at a size that spans several tiles and a ragged tail, then a smaller one: the second
    # call must not see the first one's key rows
    for (B, L, H, D, vl) in ((2, 700, 3, 64, [700, 413]), (1, 130, 2, 64, None)):
        say(f"case: jattn_fwd_noalloc B{B} L{L} H{H} D{D} valid_len={vl}")
        inp = make_shape_inputs(B, L, H, D, seed=11, valid_len=vl)
        (oa, la, ga), (ob, lb, gb) = run_both(lib, inp)
        assert torch.equal(oa, ob) and torch.equal(la, lb)
        for x, y in zip(ga, gb):
            assert torch.equal(x, y)
