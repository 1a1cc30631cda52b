"""MI355X (gfx950) library for the five bias-free decode projections out = x @ W^T.

The work runs in hand-written HIP kernels behind the C ABI of include/proj.h;
`binding` mirrors that ABI in Python (ctypes) and is imported lazily so that
host-only modules (layers, roofline) load without the built library.
"""

from . import layers, roofline  # noqa: F401

__all__ = ["layers", "roofline", "binding"]


def __getattr__(name):
    if name == "binding":
        import importlib

        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
