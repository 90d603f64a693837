"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package holds no arithmetic of the method (no rotation, no attention,
no rounding of results, no allocation policy): it only draws shapes, lengths,
block tables, run lists and N(0, 1) values from fixed seeds, shaped on the
workloads the pages describe.
"""

from .configs import CONFIGS, get_config  # noqa: F401
