"""The Python bindings fail loudly: a missing library raises instead of falling back to anything,
CPU tensors are refused before any library call, and (on a GPU) tensors of the wrong dtype, shape
or layout are refused with a message that names them."""
import pytest
import torch

from diffusion_transformer_joint_amd import _lib, adaln, mlp, ops


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libjattn.so"))
    with pytest.raises(ImportError, match="missing"):
        _lib.load()


def test_cpu_tensors_are_refused():
    q = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    g = torch.ones(2, 32)
    with pytest.raises(ValueError, match="HIP device"):
        ops.forward(q, q, q, g)
    with pytest.raises(ValueError):
        ops.forward(q[0], q[0], q[0], g)  # not [B, L, H, D]


@pytest.mark.gpu
def test_wrong_tensors_are_refused_on_the_gpu():
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16, device=dev)
    g = torch.ones(2, 32, device=dev)
    with pytest.raises(ValueError, match="k"):
        ops.forward(q, q.float(), q, g)                      # wrong dtype
    with pytest.raises(ValueError, match="v"):
        ops.forward(q, q, q[:, :4], g)                       # wrong shape
    with pytest.raises(ValueError, match="k"):
        ops.forward(q, q.transpose(1, 2).contiguous().transpose(1, 2), q, g)  # not contiguous
    with pytest.raises(ValueError, match="gains"):
        ops.forward(q, q, q, torch.ones(2, 16, device=dev))  # gains of the wrong width
    x = tuple(torch.zeros(1, n, 64, dtype=torch.bfloat16, device=dev) for n in (5, 3))
    mod = tuple(torch.zeros(1, 2, 64, device=dev) for _ in range(2))
    w = tuple(torch.zeros(3 * 64, 64, dtype=torch.bfloat16, device=dev) for _ in range(2))
    with pytest.raises(ValueError):
        adaln.adaln_qkv_forward(x, mod, (w[0], w[1][:64]), None)   # text-stream weight of the wrong shape
    w12 = tuple(torch.zeros(2 * 128, 64, dtype=torch.bfloat16, device=dev) for _ in range(2))
    w2 = tuple(torch.zeros(64, 128, dtype=torch.bfloat16, device=dev) for _ in range(2))
    wfc = tuple(torch.zeros(64, 64, dtype=torch.bfloat16, device=dev) for _ in range(2))
    with pytest.raises(ValueError):
        mlp.mlp_forward(x, x, mod, wfc, w12, (w2[0], w2[1].float()), None, None, None)  # fp32 W2
