"""HSTU layer on MI355X (gfx950): HIP kernels behind a C-ABI library.

`binding` holds the torch-facing wrappers of the C entry points declared in
include/hstu.h; `flops` the algorithmic cost model used for reporting.
"""
import importlib

from . import flops  # noqa: F401

__all__ = ["flops", "binding"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
