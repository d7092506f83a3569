"""fp64 CPU oracle of the HSTU layer -- test infrastructure only.

Imported by the test suite, by the package entry's smoke check and by the
benchmark's CPU-baseline leg, never by the HIP path.
"""
from . import hstu

__all__ = ["hstu"]
