"""Seeded synthetic inputs shared by the oracle and the GPU path (no method arithmetic)."""
from . import configs, content  # noqa: F401
