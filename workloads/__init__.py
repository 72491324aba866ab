"""Seeded synthetic inputs for the ISD step.

This package only draws random numbers and lays them out; it holds none of the
step's own arithmetic (no attention, no acceptance test, no residual sampling,
no KV commit).  Both the float64 oracle (``oracle/``) and the HIP path take
their inputs from here, so a parity test feeds the same bytes to both sides.
"""

from .configs import CONFIGS, WorkloadConfig, get_config
from .gen import Workload, make_workload, stride_rows

__all__ = ["CONFIGS", "WorkloadConfig", "get_config", "Workload", "make_workload", "stride_rows"]
