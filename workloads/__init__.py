"""Seeded synthetic inputs (counter-based RNG, storage rounding, workload shapes).

Shared by the tests, `bench.py` and the smoke check.  Holds no arithmetic of the
attention method itself.
"""
from . import rng, configs  # noqa: F401
from .configs import CONFIGS, ORDER, Config, make_inputs, make_tensor, scaled, shapes  # noqa: F401
