"""Oracle of the S3-DiT hot path (plain NumPy, CPU).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's
CPU-baseline leg, never by the library or its binding.
"""
from .zdit_oracle import *  # noqa: F401,F403
