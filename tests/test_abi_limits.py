"""Size limits of every entry-point family at their exact boundaries (host side only, no GPU): the
largest accepted size gets a workspace size, the next one is rejected (workspace size 0). The limits
keep every element index the kernels form in 32-bit arithmetic below 2^31."""
import pytest

from diffusion_transformer_joint_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_attention_limits(lib):
    # B * H * L < 2^31
    assert lib.jattn_fwd_workspace_bytes((1 << 21) - 1, 1024, 1, 32) > 0
    assert lib.jattn_fwd_workspace_bytes(1 << 21, 1024, 1, 32) == 0
    assert lib.jattn_bwd_workspace_bytes(1 << 21, 1024, 1, 32) == 0
    # (L + 256) * H * D < 2^31
    assert lib.jattn_fwd_workspace_bytes(1, (1 << 24) - 257, 1, 128) > 0
    assert lib.jattn_fwd_workspace_bytes(1, (1 << 24) - 256, 1, 128) == 0
    # the large-batch GPU test's shape is well inside
    assert lib.jattn_bwd_workspace_bytes(4096, 1024, 16, 64) > 0


def test_adaln_limits(lib):
    # T * 3C < 2^31 per stream (C = 64: T < 11184810.67)
    assert lib.jattn_adaln_qkv_fwd_workspace_bytes(1, 11184810, 0, 64) > 0
    assert lib.jattn_adaln_qkv_fwd_workspace_bytes(1, 11184811, 0, 64) == 0
    assert lib.jattn_adaln_qkv_bwd_workspace_bytes(1, 0, 11184811, 64) == 0
    # the near-limit GPU test's shape
    assert lib.jattn_adaln_qkv_fwd_workspace_bytes(1, 233000, 10, 3072) > 0
    assert lib.jattn_adaln_qkv_fwd_workspace_bytes(1, 233017, 0, 3072) == 0


def test_mlp_limits(lib):
    # T * 2F < 2^31 per stream (F = 16384: T < 65536)
    assert lib.jattn_mlp_fwd_workspace_bytes(1, 65535, 0, 64, 16384) > 0
    assert lib.jattn_mlp_fwd_workspace_bytes(1, 65536, 0, 64, 16384) == 0
    assert lib.jattn_mlp_bwd_workspace_bytes(1, 0, 65536, 64, 16384) == 0
    # T * C < 2^31 (C = 4096: T < 524288), with F small
    assert lib.jattn_mlp_fwd_workspace_bytes(1, 524287, 0, 4096, 64) > 0
    assert lib.jattn_mlp_fwd_workspace_bytes(1, 524288, 0, 4096, 64) == 0
    # the near-limit GPU test's shape
    assert lib.jattn_mlp_fwd_workspace_bytes(1, 131000, 60, 3072, 8192) > 0
