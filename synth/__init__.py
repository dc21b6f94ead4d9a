"""Seeded synthetic inputs (no arithmetic of the method)."""
from . import gen, configs  # noqa: F401
