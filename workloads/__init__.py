"""Seeded synthetic workloads for paged decode attention.

This package only draws random numbers and lays out operation traces.  It
holds none of the attention, slot or block-table arithmetic: both the CPU
oracle and the HIP path consume what it produces, and neither is imported
here.
"""

from .configs import (  # noqa: F401
    CONFIG_IDS,
    Workload,
    make_workload,
    custom_workload,
    new_token_kv,
)
