"""Plain fp64 CPU oracle of the KV-cache fusion step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path never calls it and shares no code with it.
"""
from .reference import *  # noqa: F401,F403
