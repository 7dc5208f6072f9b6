"""ctypes loader for libjattn.so (the C ABI declared in include/jattn.h, jattn_adaln.h and jattn_mlp.h).

The library is built in-tree by ``diffusion_transformer_joint_amd.build``. Loading fails loudly if it
is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjattn.so")

STATUS = {0: "JATTN_SUCCESS", 1: "JATTN_ERROR_INVALID_VALUE", 2: "JATTN_ERROR_NOT_SUPPORTED",
          3: "JATTN_ERROR_WORKSPACE", 4: "JATTN_ERROR_HIP"}
SUCCESS, INVALID_VALUE, NOT_SUPPORTED, WORKSPACE, HIP = range(5)

EXPORTED = ("jattn_fwd", "jattn_fwd_noalloc", "jattn_fwd_noalloc_max_scratch_bytes", "jattn_fwd_ex", "jattn_fwd_workspace_bytes", "jattn_bwd", "jattn_bwd_ex", "jattn_bwd_workspace_bytes",
            "jattn_fwd_streams", "jattn_bwd_streams", "jattn_varlen_fwd_workspace_bytes",
            "jattn_varlen_bwd_workspace_bytes", "jattn_fwd_varlen", "jattn_bwd_varlen", "jattn_fwd_window",
            "jattn_bwd_window", "jattn_adaln_qkv_fwd_workspace_bytes", "jattn_adaln_qkv_bwd_workspace_bytes",
            "jattn_adaln_qkv_fwd", "jattn_adaln_qkv_bwd", "jattn_mlp_fwd_workspace_bytes", "jattn_mlp_bwd_workspace_bytes",
            "jattn_mlp_fwd", "jattn_mlp_bwd", "jattn_probe_saturate", "jattn_probe_dq_accumulation", "jattn_probe_tile",
            "jattn_probe_lds_read", "jattn_probe_issue", "jattn_probe_pingpong",
            "jattn_status_string", "jattn_abi_version")
ABI_VERSION = 9
FWD_STAGES = ("prenorm_kernel", "fwd_kernel")
BWD_STAGES = ("prenorm_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "dg_reduce_kernel")
ADALN_FWD_STAGES = ("modulate_kernel", "qkv_gemm_kernel")
ADALN_BWD_STAGES = ("transpose_w_kernel", "dh_gemm_kernel", "rows_bwd_kernel", "dw_gemm_kernel", "reductions")
MLP_FWD_STAGES = ("fc_gemm", "modulate_kernel", "swiglu_gemm_kernel", "down_gemm")
MLP_BWD_STAGES = ("transpose_w_kernel", "dhid_gemm", "dw2_gemm", "du_gemm", "dw12_gemm", "rows_bwd_kernel", "do_gemm",
                  "dwfc_gemm", "reductions")

_lock = threading.Lock()
_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
F = ctypes.c_float


class JattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


def load() -> ctypes.CDLL:
    """Load libjattn.so once and declare the argument types of every entry point."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m diffusion_transformer_joint_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.jattn_fwd.restype = I
        lib.jattn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, F, P, P, P, ctypes.c_size_t, P]
        lib.jattn_fwd_noalloc.restype = I
        lib.jattn_fwd_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, F, F, P, P, P]
        lib.jattn_fwd_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
        lib.jattn_fwd_noalloc_max_scratch_bytes.argtypes = []
        lib.jattn_fwd_ex.restype = I
        lib.jattn_fwd_ex.argtypes = [P, P, P, P, P, I, I, I, I, F, F, P, P, P, ctypes.c_size_t, P, I, P]
        lib.jattn_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_fwd_workspace_bytes.argtypes = [I, I, I, I]
        lib.jattn_bwd.restype = I
        lib.jattn_bwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, F, P, P, P, P, P,
                                  ctypes.c_size_t, P, P]
        lib.jattn_bwd_ex.restype = I
        lib.jattn_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, F, P, P, P, P, P,
                                     ctypes.c_size_t, P, P, I, P]
        lib.jattn_fwd_streams.restype = I
        lib.jattn_fwd_streams.argtypes = [P, P, P, P, P, I, I, I, I, I, F, F, P, P, P, ctypes.c_size_t, P, I, P]
        lib.jattn_bwd_streams.restype = I
        lib.jattn_bwd_streams.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, F, F, P, P, P, P, P,
                                          ctypes.c_size_t, P, P, I, P]
        lib.jattn_fwd_window.restype = I
        lib.jattn_fwd_window.argtypes = [P, P, P, P, P, I, I, I, I, F, F, I, I, P, P, P, ctypes.c_size_t, P, I, P]
        lib.jattn_bwd_window.restype = I
        lib.jattn_bwd_window.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, F, I, I, P, P, P, P, P,
                                         ctypes.c_size_t, P, P, I, P]
        lib.jattn_varlen_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_varlen_fwd_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.jattn_varlen_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_varlen_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.jattn_fwd_varlen.restype = I
        lib.jattn_fwd_varlen.argtypes = [P, P, P, P, P, I, I, I, I, I, F, F, P, P, P, ctypes.c_size_t, P, I, P]
        lib.jattn_bwd_varlen.restype = I
        lib.jattn_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, F, F, P, P, P, P, P,
                                         ctypes.c_size_t, P, P, I, P]
        lib.jattn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_bwd_workspace_bytes.argtypes = [I, I, I, I]
        lib.jattn_adaln_qkv_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_adaln_qkv_fwd_workspace_bytes.argtypes = [I, I, I, I]
        lib.jattn_adaln_qkv_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_adaln_qkv_bwd_workspace_bytes.argtypes = [I, I, I, I]
        lib.jattn_adaln_qkv_fwd.restype = I
        lib.jattn_adaln_qkv_fwd.argtypes = [P, P, P, P, I, I, I, I, F, P, P, P, P, ctypes.c_size_t, P, I, P]
        lib.jattn_adaln_qkv_bwd.restype = I
        lib.jattn_adaln_qkv_bwd.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, P, P, P, ctypes.c_size_t, P,
                                            ctypes.c_size_t, P, I, P]
        lib.jattn_mlp_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_mlp_fwd_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.jattn_mlp_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.jattn_mlp_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.jattn_mlp_fwd.restype = I
        lib.jattn_mlp_fwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, P, ctypes.c_size_t, P, I, P]
        lib.jattn_probe_saturate.restype = I
        lib.jattn_probe_saturate.argtypes = [I, I, I, ctypes.c_float, P, P]
        lib.jattn_probe_dq_accumulation.restype = I
        lib.jattn_probe_dq_accumulation.argtypes = [I, I, I, I, I, P, ctypes.c_size_t, P]
        lib.jattn_probe_tile.restype = I
        lib.jattn_probe_tile.argtypes = [I, I, I, ctypes.c_float, P, P, P]
        lib.jattn_probe_lds_read.restype = I
        lib.jattn_probe_lds_read.argtypes = [I, I, I, P, P]
        lib.jattn_probe_issue.restype = I
        lib.jattn_probe_issue.argtypes = [I, I, I, ctypes.c_float, P, P, P]
        lib.jattn_probe_pingpong.restype = I
        lib.jattn_probe_pingpong.argtypes = [I, I, I, I, ctypes.c_float, P, P, P]
        lib.jattn_mlp_bwd.restype = I
        lib.jattn_mlp_bwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P,
                                      ctypes.c_size_t, P, I, P]
        lib.jattn_status_string.restype = ctypes.c_char_p
        lib.jattn_status_string.argtypes = [I]
        lib.jattn_abi_version.restype = I
        lib.jattn_abi_version.argtypes = []
        if lib.jattn_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {lib.jattn_abi_version()}, expected {ABI_VERSION}; "
                              "rebuild it")
        _lib = lib
        return lib


class PtrPair:
    """Host array of two device pointers ({image part, text part}) for the two-stream entry points.
    Keep the object alive for the duration of the call; `.arg` is what the call takes."""

    def __init__(self, a, b):
        self.arr = (ctypes.c_void_p * 2)(a, b)
        self.arg = ctypes.cast(self.arr, ctypes.c_void_p)


def event_array(events):
    """(pointer to a host array of hipEvent_t, count) for the stage-event arguments; (None, 0) for none.
    The array is kept alive on the returned pointer object for the duration of the call."""
    if not events:
        return None, 0
    for e in events:
        if not e.cuda_event:  # torch creates the hipEvent_t on the first record
            e.record()
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    ptr = ctypes.cast(arr, ctypes.c_void_p)
    ptr._keep = arr
    return ptr, len(events)


def check(fn: str, status: int) -> None:
    if status != SUCCESS:
        raise JattnError(fn, status)
