"""Seeded synthetic inputs for joint image+text attention and the adaLN-modulated QKV projection.

This module only draws random tensors with the shapes of the workloads below; it holds none of the
method's arithmetic, so both the fp64 oracles (test-side) and the HIP path can be fed from it.

Workload shapes (the pages give no dataset we can use; these tensors stand in for the activations
the models on the pages produce):

* ``tiny``      - B1 H2 D32, 4x4 patch grid (16 image tokens) + 8 text tokens = L 24.
* ``mmdit512``  - B16 H12 D64, 512 px image -> 4x64x64 latent, patch 2 -> 1024 image tokens,
                  plus 77 CLIP text tokens = L 1101 (re-diffusion README: the architecture
                  flowchart and the profiling table quote batch 16 and a B x 12 x 1101 x 1101
                  score matrix; width 768 / 12 heads gives D 64).
* ``dit256``    - B64 H16 D72, class-conditional DiT-XL/2 at 256 px: 32x32x4 latent, patch 2 ->
                  256 image tokens, no text stream (DiT-MoE README, training and sampling
                  commands name DiT-XL/2 at 256 px).
* ``mmdit768``  - B4 H24 D128, 768 px: 96x96 latent, patch 2 -> 2304 image tokens + 77 text
                  tokens = L 2381; the q, k, v rows at text positions are multiplied by 3 before
                  the bf16 cast (LavenderFlow model card: 768x768 MM-DiT).
* ``ragged``    - B2 H24 D128, 4096 image tokens + up to 256 text tokens, L 4352; per-sample
                  valid text length drawn uniformly from [1, 256]; keys past
                  valid_len[b] = 4096 + txt_len[b] are padding (diffusion-pipe summary: the
                  attention wrapper's varlen path).

Recipe (all on CPU, one ``torch.Generator`` seeded with ``seed``, in this order):
1. ragged only: ``txt_len = randint(1, 257, (B,))``.
2. q, k, v = ``randn(B, L, H, D)`` fp32 each; ``mmdit768`` scales the text rows by 3; cast to bf16.
3. gains = ``1 + 0.1 * randn(2, D)`` fp32 (row 0 for Q, row 1 for K).
4. dout = ``randn(B, L, H, D).bfloat16()``.
5. two-stream inputs only: per-stream gains = ``1 + 0.1 * randn(2, 2, D)`` fp32 ([stream][Q, K]).

Packed variable-length inputs (sequences back to back, [total, H, D], ``cu_seqlens`` offsets):

* ``varlen_ragged``   - the ``ragged`` workload without its padding: sequence b is rows
                        [0, valid_len[b]) of that workload's sequence b (same seed-0 draws).
* ``varlen_multires`` - B16 H12 D64 (the 512px model's heads), a multi-resolution batch: each
                        sample's image is a square of 256, 384, 512, 640 or 768 px (patch-2 tokens
                        of the 8x latent: 256, 576, 1024, 1600, 2304 tokens) followed by 1..77 text
                        tokens (re-diffusion README: aspect buckets at 512 base resolution, with
                        multi-resolution batching named as future work). Recipe: image size index
                        ``randint(0, 5, (B,))``, text length ``randint(1, 78, (B,))``, then q, k, v =
                        ``randn(total, H, D)`` bf16 each, gains ``1 + 0.1 * randn(2, D)``, dout
                        ``randn(total, H, D)`` bf16.
Text tokens sit at positions N_img .. L-1 (image first, text last). The two-stream inputs are the
same q, k, v and dout split along the token axis into an image part [B, N_img, H, D] and a text
part [B, N_txt, H, D] (each its own contiguous tensor).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    n_img: int
    n_txt: int
    txt_row_scale: float = 1.0
    ragged_text: bool = False

    @property
    def L(self) -> int:
        return self.n_img + self.n_txt


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, H=2, D=32, n_img=16, n_txt=8),
    "mmdit512": Workload("mmdit512", B=16, H=12, D=64, n_img=1024, n_txt=77),
    "dit256": Workload("dit256", B=64, H=16, D=72, n_img=256, n_txt=0),
    "mmdit768": Workload("mmdit768", B=4, H=24, D=128, n_img=2304, n_txt=77, txt_row_scale=3.0),
    "ragged": Workload("ragged", B=2, H=24, D=128, n_img=4096, n_txt=256, ragged_text=True),
}

EPS = 1e-6


def default_scale(D: int) -> float:
    """Softmax scale 1/sqrt(D) with the true head dim."""
    return 1.0 / math.sqrt(D)


def make_inputs(workload: str | Workload, seed: int = 0) -> dict:
    """Draw the inputs of a named workload. Returns CPU tensors:
    q, k, v, dout: bf16 [B, L, H, D]; gains: fp32 [2, D]; valid_len: int32 [B] or None;
    plus the python scalars scale, eps and the workload itself."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    return _draw(w, torch.Generator().manual_seed(seed))


def _split(t: torch.Tensor, n_img: int):
    return t[:, :n_img].contiguous(), t[:, n_img:].contiguous()


def make_stream_inputs(workload: str | Workload, seed: int = 0) -> dict:
    """Two-stream inputs of a named workload: q, k, v, dout as (image, text) pairs of bf16 tensors
    [B, N_img, H, D] and [B, N_txt, H, D]; gains fp32 [2, 2, D] (gains[s, 0] for the Q rows and
    gains[s, 1] for the K rows of stream s; image = 0, text = 1); valid_len as in make_inputs (a
    prefix length of the joint sequence, image first)."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    g = torch.Generator().manual_seed(seed)
    d = _draw(w, g)
    gains = (1.0 + 0.1 * torch.randn(2, 2, w.D, generator=g)).float()
    out = {k: _split(d[k], w.n_img) for k in ("q", "k", "v", "dout")}
    out.update(gains=gains, valid_len=d["valid_len"], scale=d["scale"], eps=d["eps"], workload=w)
    return out


def make_shape_stream_inputs(B: int, n_img: int, n_txt: int, H: int, D: int, seed: int = 0,
                             valid_len: Optional[list] = None, scale: Optional[float] = None,
                             eps: float = EPS, gain_std: float = 0.1) -> dict:
    """Two-stream inputs of an arbitrary shape (edge-case tests): the make_shape_inputs recipe for the
    joint sequence, split at n_img, then per-stream gains 1 + gain_std * randn(2, 2, D)."""
    L = n_img + n_txt
    g = torch.Generator().manual_seed(seed)
    joint = [torch.randn(B, L, H, D, generator=g).bfloat16() for _ in range(3)]
    dout = torch.randn(B, L, H, D, generator=g).bfloat16()
    gains = (1.0 + gain_std * torch.randn(2, 2, D, generator=g)).float()
    vl = None if valid_len is None else torch.tensor(valid_len, dtype=torch.int32)
    w = Workload(f"B{B}I{n_img}T{n_txt}H{H}D{D}", B=B, H=H, D=D, n_img=n_img, n_txt=n_txt)
    return dict(q=_split(joint[0], n_img), k=_split(joint[1], n_img), v=_split(joint[2], n_img),
                dout=_split(dout, n_img), gains=gains, valid_len=vl,
                scale=default_scale(D) if scale is None else float(scale), eps=eps, workload=w)


def _draw(w: Workload, g: torch.Generator) -> dict:
    B, L, H, D = w.B, w.L, w.H, w.D
    valid_len = None
    if w.ragged_text:
        txt_len = torch.randint(1, w.n_txt + 1, (B,), generator=g)
        valid_len = (w.n_img + txt_len).to(torch.int32)
    qkv = []
    for _ in range(3):
        x = torch.randn(B, L, H, D, generator=g)
        if w.txt_row_scale != 1.0 and w.n_txt > 0:
            x[:, w.n_img:] *= w.txt_row_scale
        qkv.append(x.bfloat16())
    gains = 1.0 + 0.1 * torch.randn(2, D, generator=g)
    dout = torch.randn(B, L, H, D, generator=g).bfloat16()
    return dict(q=qkv[0], k=qkv[1], v=qkv[2], gains=gains.float(), dout=dout,
                valid_len=valid_len, scale=default_scale(D), eps=EPS, workload=w)


def make_shape_inputs(B: int, L: int, H: int, D: int, seed: int = 0,
                      valid_len: Optional[list] = None, scale: Optional[float] = None,
                      eps: float = EPS, gain_std: float = 0.1, qk_std: float = 1.0) -> dict:
    """Same recipe for an arbitrary shape (edge-case tests). ``valid_len`` is taken as given."""
    g = torch.Generator().manual_seed(seed)
    q = (qk_std * torch.randn(B, L, H, D, generator=g)).bfloat16()
    k = (qk_std * torch.randn(B, L, H, D, generator=g)).bfloat16()
    v = torch.randn(B, L, H, D, generator=g).bfloat16()
    gains = (1.0 + gain_std * torch.randn(2, D, generator=g)).float()
    dout = torch.randn(B, L, H, D, generator=g).bfloat16()
    vl = None if valid_len is None else torch.tensor(valid_len, dtype=torch.int32)
    return dict(q=q, k=k, v=v, gains=gains, dout=dout, valid_len=vl,
                scale=default_scale(D) if scale is None else float(scale), eps=eps,
                workload=Workload(f"B{B}L{L}H{H}D{D}", B=B, H=H, D=D, n_img=L, n_txt=0))


def flops(B: int, L: int, H: int, D: int, valid_len=None) -> dict:
    """Algorithmic FLOPs: forward 4*D per (query, valid key) pair, backward 2.5x that."""
    if valid_len is None:
        pairs = B * L * L
    else:
        pairs = sum(L * max(0, min(L, int(n))) for n in valid_len)
    fwd = 4.0 * H * D * pairs
    return dict(fwd=fwd, bwd=2.5 * fwd, total=3.5 * fwd,
                fwd_padded=4.0 * B * H * L * L * D)


# ------------------------------------------------------------------------------------------------
# Packed variable-length inputs

MULTIRES_IMG_TOKENS = (256, 576, 1024, 1600, 2304)  # 256 .. 768 px squares, 16 px per token


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    B: int
    H: int
    D: int


VARLEN_WORKLOADS: Dict[str, VarlenWorkload] = {
    "varlen_ragged": VarlenWorkload("varlen_ragged", B=2, H=24, D=128),
    "varlen_multires": VarlenWorkload("varlen_multires", B=16, H=12, D=64),
}


def _pack(seqs):
    return torch.cat(seqs, dim=0).contiguous()


def make_varlen_inputs(workload: str, seed: int = 0) -> dict:
    """Packed inputs of a named variable-length workload. Returns CPU tensors q, k, v, dout bf16
    [total, H, D]; gains fp32 [2, D]; cu_seqlens int32 [B + 1]; plus lengths, max_seqlen, scale, eps
    and the workload."""
    w = VARLEN_WORKLOADS[workload]
    if workload == "varlen_ragged":
        d = make_inputs("ragged", seed=seed)
        lengths = d["valid_len"].tolist()
        t = {k: _pack([d[k][b, :n] for b, n in enumerate(lengths)]) for k in ("q", "k", "v", "dout")}
        gains = d["gains"]
    else:
        g = torch.Generator().manual_seed(seed)
        size = torch.randint(0, len(MULTIRES_IMG_TOKENS), (w.B,), generator=g)
        txt = torch.randint(1, 78, (w.B,), generator=g)
        lengths = [MULTIRES_IMG_TOKENS[int(i)] + int(n) for i, n in zip(size, txt)]
        total = sum(lengths)
        qkv = [torch.randn(total, w.H, w.D, generator=g).bfloat16() for _ in range(3)]
        gains = (1.0 + 0.1 * torch.randn(2, w.D, generator=g)).float()
        dout = torch.randn(total, w.H, w.D, generator=g).bfloat16()
        t = dict(q=qkv[0], k=qkv[1], v=qkv[2], dout=dout)
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    return dict(q=t["q"], k=t["k"], v=t["v"], dout=t["dout"], gains=gains, cu_seqlens=cu, lengths=lengths,
                max_seqlen=max(lengths), scale=default_scale(w.D), eps=EPS, workload=w)


def make_shape_varlen_inputs(lengths, H: int, D: int, seed: int = 0, scale: Optional[float] = None,
                             eps: float = EPS, gain_std: float = 0.1) -> dict:
    """Packed inputs of given sequence lengths (edge-case tests): q, k, v = randn(total, H, D) bf16,
    gains 1 + gain_std * randn(2, D), dout randn bf16, in that order."""
    g = torch.Generator().manual_seed(seed)
    total = int(sum(lengths))
    qkv = [torch.randn(total, H, D, generator=g).bfloat16() for _ in range(3)]
    gains = (1.0 + gain_std * torch.randn(2, D, generator=g)).float()
    dout = torch.randn(total, H, D, generator=g).bfloat16()
    cu = torch.tensor([0] + list(torch.tensor(list(lengths)).cumsum(0).tolist()), dtype=torch.int32)
    w = VarlenWorkload(f"varlen{list(lengths)}H{H}D{D}", B=len(lengths), H=H, D=D)
    return dict(q=qkv[0], k=qkv[1], v=qkv[2], dout=dout, gains=gains, cu_seqlens=cu, lengths=list(lengths),
                max_seqlen=max(max(lengths), 1), scale=default_scale(D) if scale is None else float(scale), eps=eps,
                workload=w)


def varlen_flops(lengths, H: int, D: int) -> dict:
    """Algorithmic FLOPs of a packed batch: 4*D per (query, key) pair of each sequence, backward 2.5x."""
    pairs = sum(int(n) * int(n) for n in lengths)
    fwd = 4.0 * H * D * pairs
    return dict(fwd=fwd, bwd=2.5 * fwd, total=3.5 * fwd)


# ------------------------------------------------------------------------------------------------
# adaLN-modulated QKV projection (one call covers the image and the text stream of a layer)
#
# * ``mmdit512`` - B16, 1024 image + 77 text tokens, C = 768 (12 heads x 64): the 512 px model.
# * ``mmdit768`` - B4, 2304 image + 77 text tokens, C = 3072 (24 heads x 128): the 768 px model.
#
# Recipe (one CPU generator seeded with ``seed``; for the image stream, then the text stream):
#   x = randn(B, n_s, C).bfloat16();  mod = 0.2 * randn(B, 2, C) (fp32; row 0 shift, row 1 scale);
#   w = ((2 rand(3C, C) - 1) / sqrt(C)).bfloat16()  and  bias = (2 rand(3C) - 1) / sqrt(C)  (torch's
#   default Linear initialisation); dq, dk, dv = randn(B, n_s, C).bfloat16() each.
# The modulation is zero at initialisation in the models on the pages and grows in training; 0.2
# makes both of its terms matter in the tests.

@dataclass(frozen=True)
class AdalnWorkload:
    name: str
    B: int
    n_img: int
    n_txt: int
    C: int


ADALN_WORKLOADS = {
    "mmdit512": AdalnWorkload("mmdit512", B=16, n_img=1024, n_txt=77, C=768),
    "mmdit768": AdalnWorkload("mmdit768", B=4, n_img=2304, n_txt=77, C=3072),
}


def make_adaln_inputs(B: int, n_img: int, n_txt: int, C: int, seed: int = 0, mod_std: float = 0.2) -> dict:
    g = torch.Generator().manual_seed(seed)
    out = {k: [] for k in ("x", "mod", "w", "bias", "dq", "dk", "dv")}
    for n in (n_img, n_txt):
        out["x"].append(torch.randn(B, n, C, generator=g).bfloat16())
        out["mod"].append(mod_std * torch.randn(B, 2, C, generator=g))
        out["w"].append(((2 * torch.rand(3 * C, C, generator=g) - 1) / math.sqrt(C)).bfloat16())
        out["bias"].append((2 * torch.rand(3 * C, generator=g) - 1) / math.sqrt(C))
        for key in ("dq", "dk", "dv"):
            out[key].append(torch.randn(B, n, C, generator=g).bfloat16())
    res = {k: tuple(v) for k, v in out.items()}
    res.update(B=B, n_img=n_img, n_txt=n_txt, C=C, eps=EPS)
    return res


def make_workload_adaln_inputs(name: str, seed: int = 0) -> dict:
    w = ADALN_WORKLOADS[name]
    return make_adaln_inputs(w.B, w.n_img, w.n_txt, w.C, seed=seed)


def adaln_flops(B: int, n_img: int, n_txt: int, C: int) -> dict:
    """Algorithmic FLOPs of the projection GEMMs: forward 2 T C 3C (T = all tokens of both streams);
    backward twice that (dh = dY W and dW = dY^T h). The elementwise LayerNorm work is not counted."""
    T = B * (n_img + n_txt)
    fwd = 2.0 * T * C * 3 * C
    return {"fwd": fwd, "bwd": 2 * fwd, "total": 3 * fwd}


# ------------------------------------------------------------------------------------------------
# MLP block after the attention (fc, adaLN, SwiGLU, one residual; both streams per call)
#
# * ``mmdit512`` - B16, 1024 image + 77 text tokens, C = 768, hidden F = 2048 (8C/3: the SwiGLU width
#                  with the parameters of a 4C GELU MLP; the pages give no width).
# * ``mmdit768`` - B4, 2304 image + 77 text tokens, C = 3072, F = 8192.
#
# Recipe (one CPU generator seeded with ``seed``; image stream, then text stream): o, x =
# randn(B, n_s, C).bfloat16() each; mod = 0.2 * randn(B, 2, C); wfc = U(+-1/sqrt C) [C, C] bf16,
# bfc = U(+-1/sqrt C) [C]; w12 = U(+-1/sqrt C) [2F, C] bf16, b12 = U(+-1/sqrt C) [2F]; w2 = U(+-1/sqrt F)
# [C, F] bf16, b2 = U(+-1/sqrt F) [C] (torch's default Linear initialisation); dout =
# randn(B, n_s, C).bfloat16().

@dataclass(frozen=True)
class MlpWorkload:
    name: str
    B: int
    n_img: int
    n_txt: int
    C: int
    F: int


MLP_WORKLOADS = {
    "mmdit512": MlpWorkload("mmdit512", B=16, n_img=1024, n_txt=77, C=768, F=2048),
    "mmdit768": MlpWorkload("mmdit768", B=4, n_img=2304, n_txt=77, C=3072, F=8192),
}


def make_mlp_inputs(B: int, n_img: int, n_txt: int, C: int, F: int, seed: int = 0, mod_std: float = 0.2) -> dict:
    g = torch.Generator().manual_seed(seed)
    u = lambda shape, fan: (2 * torch.rand(*shape, generator=g) - 1) / math.sqrt(fan)
    keys = ("o", "x", "mod", "wfc", "bfc", "w12", "b12", "w2", "b2", "dout")
    out = {k: [] for k in keys}
    for n in (n_img, n_txt):
        out["o"].append(torch.randn(B, n, C, generator=g).bfloat16())
        out["x"].append(torch.randn(B, n, C, generator=g).bfloat16())
        out["mod"].append(mod_std * torch.randn(B, 2, C, generator=g))
        out["wfc"].append(u((C, C), C).bfloat16())
        out["bfc"].append(u((C,), C))
        out["w12"].append(u((2 * F, C), C).bfloat16())
        out["b12"].append(u((2 * F,), C))
        out["w2"].append(u((C, F), F).bfloat16())
        out["b2"].append(u((C,), F))
        out["dout"].append(torch.randn(B, n, C, generator=g).bfloat16())
    res = {k: tuple(v) for k, v in out.items()}
    res.update(B=B, n_img=n_img, n_txt=n_txt, C=C, F=F, eps=EPS)
    return res


def make_workload_mlp_inputs(name: str, seed: int = 0) -> dict:
    w = MLP_WORKLOADS[name]
    return make_mlp_inputs(w.B, w.n_img, w.n_txt, w.C, w.F, seed=seed)


def mlp_flops(B: int, n_img: int, n_txt: int, C: int, F: int) -> dict:
    """Algorithmic FLOPs of the block's GEMMs: forward 2 T (C^2 + 2 C F + F C) for T tokens of both
    streams (fc, gate/up, down); backward twice that (input and weight gradients of each)."""
    T = B * (n_img + n_txt)
    fwd = 2.0 * T * (C * C + 3 * C * F)
    return {"fwd": fwd, "bwd": 2 * fwd, "total": 3 * fwd}
