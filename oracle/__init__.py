"""NVFP4 reference oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP product path does not import it, and it imports nothing
from the product path.
"""
from .oracle import *  # noqa: F401,F403
