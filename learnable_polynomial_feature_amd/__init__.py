"""MI355X-native LLoPS (learnable low-rank polynomial sketch) linear attention.

The compute path is the HIP library ``libllops.so`` (C ABI in include/llops.h);
this package holds its ctypes binding and the seeded workload generator.
Importing the package does not load the library; the first binding call does,
and it raises if the library is missing.
"""
_BINDING = ("llops_featmap", "llops_featmap_bwd", "llops_linattn_fwd", "llops_linattn_causal_fwd",
            "llops_linattn_causal_bwd", "llops_linattn_bwd",
            "llops_decode_step", "llops_linattn_gated_causal_fwd", "llops_gated_decode_step",
            "llops_linattn_gated_causal_bwd",
            "llops_linattn_causal_bwd_state",
            "llops_linattn_gated_causal_bwd_state",
            "llops_workspace_bytes", "LlopsError", "library")


def __getattr__(name):
    if name in _BINDING:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
