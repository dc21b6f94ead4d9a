"""One rank's share of a Ulysses sequence-parallel attention layer on MI355X (gfx950).

The compute path is the HIP library libulysses_sp.so (C ABI declared in
include/ulysses_sp.h); `ops` wraps its entry points for torch tensors.
"""
from . import _lib, ops  # noqa: F401
from ._lib import SPError  # noqa: F401

__all__ = ["ops", "SPError"]
