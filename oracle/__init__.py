"""CPU oracle for packed-KV quantization and decode attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke entry
point and by the benchmark's CPU-baseline leg.  The GPU library never loads it.
"""
from .oracle import *  # noqa: F401,F403
