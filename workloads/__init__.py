"""Seeded synthetic inputs shared by the tests, the oracle runs and bench.py.

This package draws random numbers and lays them out; it holds none of the
compose method's arithmetic (no spans, scans, inverses or descriptors).
"""
from .gen import (Batch, CONFIGS, make_batch, make_values, random_batch,  # noqa: F401
                  staging_cap_for)
