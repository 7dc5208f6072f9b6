"""fp64 CPU oracles for QK-RMSNorm joint attention, the adaLN-modulated QKV projection and the MLP block. TEST
INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU-baseline leg, never by
the HIP library or its binding."""
from .adaln_oracle import adaln_qkv_backward, adaln_qkv_forward, adaln_qkv_fwd_bwd, layer_norm_rows
from .mlp_oracle import mlp_backward, mlp_forward, mlp_fwd_bwd
from .jattn_oracle import (attention_backward, attention_forward, attention_fwd_bwd, head_backward,
                           head_forward, rmsnorm, streams_fwd_bwd, varlen_fwd_bwd)

__all__ = ["rmsnorm", "head_forward", "head_backward", "attention_forward", "attention_backward",
           "attention_fwd_bwd", "streams_fwd_bwd", "varlen_fwd_bwd", "layer_norm_rows", "adaln_qkv_forward",
           "adaln_qkv_backward", "adaln_qkv_fwd_bwd", "mlp_forward", "mlp_backward", "mlp_fwd_bwd"]
