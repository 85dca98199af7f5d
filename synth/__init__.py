"""Seeded synthetic inputs for the TwELL sparse gated-FFN forward.

This package is shared by the tests, the benchmark and the smoke check. It
draws inputs only: it holds none of the method's arithmetic (no gate GEMM, no
ReLU, no packing, no FFN), so neither the oracle nor the HIP path depends on
the other through it.
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    Inputs,
    Workload,
    make_inputs,
    make_upstream_grad,
    scaled,
    sweep_workloads,
)
