"""MI355X (gfx950) sparse-MoE block: HIP kernels behind a C ABI (include/moe.h).

`_lib` is the ctypes binding (one function per C entry point, same names);
`layer.MoELayer` keeps a layer's weights and workspace in device memory and
calls those entry points.  Build the library first:
    python -m mixture_experts_decode_router_amd.build
"""
from . import _lib  # noqa: F401
from ._lib import MoEError, lib  # noqa: F401

__all__ = ["MoEError", "lib", "MoELayer"]


def __getattr__(name):
    # torch is only needed for the device-memory helper
    if name == "MoELayer":
        from .layer import MoELayer
        return MoELayer
    raise AttributeError(name)
