"""MI355X-native QK-RMSNorm joint image+text attention (forward and backward) on gfx950.

The compute runs in the hand-written HIP kernels of ``libjattn.so`` (C ABI, ``include/jattn.h``).
This package only marshals arguments: ``forward``, ``backward`` and the ``JointAttention`` autograd
function load the library on first use and raise if it is missing -- there is no fallback path.
"""
__all__ = ["forward", "backward", "JointAttention", "joint_attention", "workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
