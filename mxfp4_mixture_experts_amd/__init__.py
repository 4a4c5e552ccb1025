"""MI355X-native MXFP4 mixture-of-experts expert projection.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libmxfp4_moe.so``, built from ``csrc/``).  ``binding`` marshals torch
tensors into that ABI; it does no arithmetic of its own.  ``synthetic`` draws
the seeded inputs.

The binding is imported lazily so that the input generator can be used on a
machine without the library; calling any entry point without the library
raises.
"""

__all__ = ["mxfp4_moe_route_group", "mxfp4_expert_proj", "mxfp4_expert_proj_workspace_size", "moe_combine",
           "mxfp4_expert_proj_swiglu", "mxfp4_expert_proj_combine", "mxfp4_moe_decode", "mxfp4_moe_decode_swiglu",
           "mxfp4_moe_router", "mxfp4_moe_dense_route", "mxfp4_dequantize", "mxfp4_expert_proj_noalloc",
           "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
