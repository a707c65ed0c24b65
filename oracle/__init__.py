"""Independent fp64 CPU oracle for one GPU's share of context-parallel
attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library in ``sequence_context_parallelism_amd`` and neither imports the
other.  ``attention`` holds the definition (forward, LSE, merge, backward, tile
classes); ``schedule`` holds the zigzag sharding and the ring / Ulysses / USP
emulations built from it.
"""
from . import attention, schedule  # noqa: F401
