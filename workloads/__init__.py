"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.  Holds no NVFP4 arithmetic: only random draws, BF16 storage
conversion and MoE routing bookkeeping."""
from .generators import *  # noqa: F401,F403
