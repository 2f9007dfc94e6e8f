"""fp64 CPU oracle of the KroQuant online activation quantizer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.
"""
from .oracle import *  # noqa: F401,F403
