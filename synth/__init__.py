"""Seeded synthetic workloads (geometry presets + input/weight generator).

Shared by the oracle tests and the GPU tests / bench; holds no step of the
draft pass itself.
"""
from . import configs, gen  # noqa: F401
