"""HSTU layer on MI355X (gfx950): HIP kernels behind a C-ABI library."""
from . import flops  # noqa: F401
