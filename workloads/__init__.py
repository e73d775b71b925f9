"""Seeded synthetic workloads for the KV-cache fusion step.

This package only draws random inputs and lays out the chunk tables that a
caller would hand to the fusion step. It holds none of the method's arithmetic
(no rotary embedding, no softmax, no selection): the oracle and the HIP path both
consume exactly the arrays produced here.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import Workload, make_workload, make_custom  # noqa: F401
