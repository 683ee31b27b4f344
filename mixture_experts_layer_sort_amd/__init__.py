"""MI355X (gfx950) dropless top-k Mixture-of-Experts SwiGLU layer.

The layer runs in a HIP library (``libmoe_mi355x.so``, C ABI in
``include/moe.h``); this package holds its ctypes binding (``_lib``), the
buffer-owning runner and autograd function (``layer``) and the build script
(``build``).
"""
from . import _lib  # noqa: F401
from ._lib import MoEError, lib  # noqa: F401

__all__ = ["MoEError", "lib", "MoELayerRunner", "MoEFunction", "moe_layer"]


def __getattr__(name):
    if name in ("MoELayerRunner", "MoEFunction", "moe_layer"):
        from . import layer
        return getattr(layer, name)
    raise AttributeError(name)
