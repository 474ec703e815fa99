"""Seeded synthetic inputs for the paged decode workloads.

This package only draws numbers (context lengths, block orders, q/K/V values)
and rounds them to their storage type.  It holds none of the attention,
append or bookkeeping arithmetic; both the oracle side and the HIP side of
every test and of the benchmark take their inputs from here.
"""
from .configs import CONFIGS, MQ_CONFIGS, Config, MQConfig  # noqa: F401
