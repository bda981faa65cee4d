"""Seeded synthetic inputs for the Quest decode workloads."""
from .workloads import *  # noqa: F401,F403
