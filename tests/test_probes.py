"""The measurement probes of include/jattn_diag.h on the GPU, at tiny sizes: every mode launches, keeps its
per-thread outputs finite and reports a positive cycle count per wave; the dQ-accumulation probe's atomic
mode adds exactly nkb ones into every element and its partial and reduce modes give the same sums.
(Their host-side refusals are in test_abi.py; bench.py --probe-tile and --probe-dq-accumulation time them.)"""
import ctypes

import pytest
import torch

from diffusion_transformer_joint_amd import _lib

pytestmark = pytest.mark.gpu

SEED = ctypes.c_float(1e-3)


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("which", [0, 1])
def test_probe_saturate(lib, which):
    say(f"case: probe_saturate which={which} blocks=4 iters=2")
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    _lib.check("jattn_probe_saturate", lib.jattn_probe_saturate(which, 4, 2, ctypes.c_float(1.0), out.data_ptr(),
                                                                stream()))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("mode", range(8))
def test_probe_tile(lib, mode):
    say(f"case: probe_tile mode={mode} blocks=4 iters=3")
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    cyc = torch.zeros(4 * 4, dtype=torch.int64, device="cuda:0")
    _lib.check("jattn_probe_tile", lib.jattn_probe_tile(mode, 4, 3, SEED, out.data_ptr(), cyc.data_ptr(), stream()))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (cyc > 0).all()


@pytest.mark.parametrize("mode", range(3))
def test_probe_lds_read(lib, mode):
    say(f"case: probe_lds_read mode={mode} blocks=4 iters=3")
    cyc = torch.zeros(4 * 4, dtype=torch.int64, device="cuda:0")
    _lib.check("jattn_probe_lds_read", lib.jattn_probe_lds_read(mode, 4, 3, cyc.data_ptr(), stream()))
    torch.cuda.synchronize()
    assert (cyc > 0).all()


@pytest.mark.parametrize("mode", range(7))
def test_probe_issue(lib, mode):
    say(f"case: probe_issue mode={mode} blocks=2 iters=3")
    out = torch.full((2 * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
    cyc = torch.zeros(2 * 8, dtype=torch.int64, device="cuda:0")
    _lib.check("jattn_probe_issue", lib.jattn_probe_issue(mode, 2, 3, SEED, out.data_ptr(), cyc.data_ptr(), stream()))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (cyc > 0).all()


@pytest.mark.parametrize("mode", range(3))
@pytest.mark.parametrize("lds", [0, 1])
def test_probe_pingpong(lib, mode, lds):
    say(f"case: probe_pingpong mode={mode} lds={lds} blocks=2 iters=3")
    out = torch.full((2 * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
    cyc = torch.zeros(2 * 8, dtype=torch.int64, device="cuda:0")
    _lib.check("jattn_probe_pingpong", lib.jattn_probe_pingpong(mode, lds, 2, 3, SEED, out.data_ptr(), cyc.data_ptr(),
                                                                stream()))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (cyc > 0).all()


def test_probe_dq_accumulation_sums(lib):
    pairs, L, D, nkb = 3, 100, 72, 5
    n = pairs * L * D
    say(f"case: probe_dq_accumulation pairs={pairs} L={L} D={D} nkb={nkb}")
    acc = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    _lib.check("jattn_probe_dq_accumulation",
               lib.jattn_probe_dq_accumulation(0, pairs, L, D, nkb, acc.data_ptr(), acc.numel() * 4, stream()))
    torch.cuda.synchronize()
    assert torch.equal(acc, torch.full_like(acc, float(nkb)))
    part = torch.full(((nkb + 1) * n,), float("nan"), dtype=torch.float32, device="cuda:0")
    _lib.check("jattn_probe_dq_accumulation",
               lib.jattn_probe_dq_accumulation(1, pairs, L, D, nkb, part.data_ptr(), part.numel() * 4, stream()))
    _lib.check("jattn_probe_dq_accumulation",
               lib.jattn_probe_dq_accumulation(2, pairs, L, D, nkb, part.data_ptr(), part.numel() * 4, stream()))
    torch.cuda.synchronize()
    assert torch.equal(part[: nkb * n], torch.ones(nkb * n, device="cuda:0"))
    assert torch.equal(part[nkb * n:], acc)
