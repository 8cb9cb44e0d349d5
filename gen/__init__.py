"""Seeded synthetic inputs shared by the tests, the oracle checks and the bench."""
from . import workloads  # noqa: F401
