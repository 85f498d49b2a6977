"""Seeded synthetic inputs (no step of the method lives here): workload registry and generators."""
from . import configs, gen  # noqa: F401
