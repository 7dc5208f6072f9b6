"""fp64 CPU oracle for QK-RMSNorm joint attention. TEST INFRASTRUCTURE ONLY: imported by tests,
the smoke check and the benchmark's CPU-baseline leg, never by the HIP library or its binding."""
from .jattn_oracle import (attention_backward, attention_forward, attention_fwd_bwd, head_backward,
                           head_forward, rmsnorm, streams_fwd_bwd, varlen_fwd_bwd)

__all__ = ["rmsnorm", "head_forward", "head_backward", "attention_forward", "attention_backward",
           "attention_fwd_bwd", "streams_fwd_bwd", "varlen_fwd_bwd"]
