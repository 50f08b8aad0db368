"""Seeded synthetic inputs (no step of the MoE method lives here)."""
from . import gen, configs  # noqa: F401
