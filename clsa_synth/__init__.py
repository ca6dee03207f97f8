"""Seeded synthetic inputs shared by the oracle and the GPU path (values only, no method arithmetic)."""
from . import gen
from .workload import Workload, config, custom

__all__ = ["gen", "Workload", "config", "custom"]
