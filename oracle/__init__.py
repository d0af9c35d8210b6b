"""CPU oracle for the store-h looped decode step (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg use this package; the HIP library never imports, links or calls it.
"""
from .looped import *  # noqa: F401,F403
from .looped import argmax_lowest  # noqa: F401
