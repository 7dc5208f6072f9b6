"""Seeded workload generators: shapes, dtypes, determinism and the ragged lengths."""
import torch

from diffusion_transformer_joint_amd.inputs import WORKLOADS, flops, make_inputs


def test_tiny_shapes_and_determinism():
    a = make_inputs("tiny", seed=0)
    b = make_inputs("tiny", seed=0)
    assert a["q"].shape == (1, 24, 2, 32) and a["q"].dtype == torch.bfloat16
    assert a["gains"].shape == (2, 32) and a["gains"].dtype == torch.float32
    assert a["valid_len"] is None
    for key in ("q", "k", "v", "gains", "dout"):
        assert torch.equal(a[key], b[key])
    assert abs(a["scale"] - 32 ** -0.5) < 1e-15 and a["eps"] == 1e-6


def test_workload_lengths():
    assert WORKLOADS["mmdit512"].L == 1101
    assert WORKLOADS["dit256"].L == 256
    assert WORKLOADS["mmdit768"].L == 2381
    assert WORKLOADS["ragged"].L == 4352


def test_ragged_valid_lengths_seed0():
    # txt_len ~ U[1, 256] drawn first from the seed-0 generator: (173, 48) -> 4096 + txt_len
    g = torch.Generator().manual_seed(0)
    txt = torch.randint(1, 257, (2,), generator=g)
    assert txt.tolist() == [173, 48]
    w = WORKLOADS["ragged"]
    small = type(w)("r", B=2, H=1, D=8, n_img=4096, n_txt=256, ragged_text=True)
    assert make_inputs(small)["valid_len"].tolist() == [4269, 4144]


def test_text_rows_scaled_in_768_workload():
    w = WORKLOADS["mmdit768"]
    small = type(w)("s", B=1, H=1, D=8, n_img=6, n_txt=3, txt_row_scale=3.0)
    ref = type(w)("r", B=1, H=1, D=8, n_img=6, n_txt=3)
    a, b = make_inputs(small), make_inputs(ref)
    assert torch.equal(a["q"][:, :6], b["q"][:, :6])
    # text rows are 3x the unscaled draw, up to the two bf16 roundings
    assert torch.allclose(a["q"][:, 6:].float(), 3 * b["q"][:, 6:].float(), rtol=1e-2)


def test_flop_count():
    f = flops(16, 1101, 12, 64)
    assert abs(f["total"] - 208.537e9) / 208.537e9 < 1e-4
    r = flops(2, 4352, 24, 128, valid_len=[4269, 4144])
    assert r["fwd"] < r["fwd_padded"]


def test_stream_inputs_split_the_joint_draw():
    from diffusion_transformer_joint_amd.inputs import make_stream_inputs
    a, b = make_inputs("tiny", seed=0), make_stream_inputs("tiny", seed=0)
    for key in ("q", "k", "v", "dout"):
        img, txt = b[key]
        assert img.shape == (1, 16, 2, 32) and txt.shape == (1, 8, 2, 32)
        assert img.is_contiguous() and txt.is_contiguous()
        assert torch.equal(torch.cat([img, txt], dim=1), a[key])
    assert b["gains"].shape == (2, 2, 32) and b["gains"].dtype == torch.float32
    assert not torch.equal(b["gains"][0], b["gains"][1])


def test_varlen_inputs():
    from diffusion_transformer_joint_amd.inputs import make_varlen_inputs, MULTIRES_IMG_TOKENS
    r = make_varlen_inputs("varlen_ragged")
    p = make_inputs("ragged")
    assert r["lengths"] == p["valid_len"].tolist() == [4269, 4144]
    assert r["cu_seqlens"].tolist() == [0, 4269, 8413] and r["cu_seqlens"].dtype == torch.int32
    assert torch.equal(r["q"][4269:], p["q"][1, :4144]) and torch.equal(r["dout"][:4269], p["dout"][0, :4269])
    m = make_varlen_inputs("varlen_multires")
    assert m["q"].shape == (sum(m["lengths"]), 12, 64) and m["max_seqlen"] == max(m["lengths"])
    assert all(1 <= n - t <= 77 for n in m["lengths"] for t in [max(x for x in MULTIRES_IMG_TOKENS if x < n)])
