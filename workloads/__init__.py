"""Seeded synthetic inputs for the Relation operator.

This module draws random numbers and applies the upstream rotary encoding for
the RoPE workload; it holds none of the Relation arithmetic. Both the oracle
side (tests, CPU baseline) and the HIP side (tests, bench) take their inputs
from here, so both see the same values.
"""
from .gen import *  # noqa: F401,F403
