"""CPU fp64 oracle (test infrastructure only; never imported by the library)."""
from . import ref  # noqa: F401
