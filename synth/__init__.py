"""Seeded synthetic inputs shared by the oracle side and the HIP side."""
from .workloads import *  # noqa: F401,F403
