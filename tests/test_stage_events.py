"""GPU test of the per-stage timing hooks of the joint backward (jattn_bwd_ex): an event array whose
first entries are NULL records only the events that are set, the results are bitwise those of
jattn_bwd, and the recorded events bracket the stage they follow (positive elapsed time)."""
import ctypes

import pytest
import torch

from diffusion_transformer_joint_amd import _lib, ops
from diffusion_transformer_joint_amd.inputs import make_shape_inputs

pytestmark = pytest.mark.gpu


def test_bwd_ex_null_stage_events():
    B, L, H, D = 2, 300, 2, 64
    print(f"case: bwd_ex with NULL stage events, B{B} L{L} H{H} D{D}, seed 4242", flush=True)
    inp = make_shape_inputs(B, L, H, D, seed=4242, valid_len=[300, 171])
    dev = torch.device("cuda:0")
    q, k, v, dout = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    gains, vl = inp["gains"].to(dev), inp["valid_len"].to(dev)
    scale, eps = inp["scale"], inp["eps"]
    out, lse = ops.forward(q, k, v, gains, vl, scale, eps)
    ref = ops.backward(q, k, v, gains, out, lse, dout, vl, scale, eps)

    lib = _lib.load()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty(2, D, dtype=torch.float32, device=dev)
    ws = torch.empty(max(int(lib.jattn_bwd_workspace_bytes(B, L, H, D)), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    before = torch.cuda.Event(enable_timing=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record(stream)  # creates the underlying events
    torch.cuda.synchronize()
    # stages: key normalisation, dq, dk/dv, gain reduction; events only after dq and after dk/dv
    arr = (ctypes.c_void_p * 3)(None, ev[0].cuda_event, ev[1].cuda_event)
    before.record(stream)
    st = lib.jattn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), gains.data_ptr(), vl.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), dout.data_ptr(), B, L, H, D, ctypes.c_float(scale), ctypes.c_float(eps),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dg.data_ptr(), ws.data_ptr(), ws.numel(),
                          None, ctypes.cast(arr, ctypes.c_void_p), 3, stream.cuda_stream)
    assert st == 0, _lib.load().jattn_status_string(st)
    torch.cuda.synchronize()
    for got, want in zip((dq, dk, dv, dg), ref):
        assert torch.equal(got, want)
    assert before.elapsed_time(ev[0]) > 0.0  # key normalisation and dq
    assert ev[0].elapsed_time(ev[1]) > 0.0  # dk/dv
