"""Seeded synthetic inputs shared by the tests, the oracle runs and bench.py.

This package draws random numbers and lays them out; it holds none of the
compose method's arithmetic (no spans, scans, inverses or descriptors).
"""
from .gen import (Batch, CONFIGS, INDEX_ROW_BYTES, make_batch, make_values,  # noqa: F401
                  random_batch, staging_cap_for)
