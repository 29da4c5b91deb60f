"""Seeded synthetic video-shaped attention inputs.

This package only draws inputs.  It holds none of the attention method's
arithmetic (no partitioning, routing, sparse execution or fitting) and is the
one module that both the CPU oracle and the GPU path may share.
"""

from .generator import (  # noqa: F401
    WORKLOADS,
    Workload,
    f90_fraction,
    make_video_qkv,
    make_workload_inputs,
    workload,
)
