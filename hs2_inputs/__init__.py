"""Seeded synthetic inputs for the HySparse2 attention hot path.

This package only draws random numbers and rounds them into the storage
formats the path consumes (fp32, bf16, FP8-e4m3 codes with per-token fp32
scales). It holds none of the method's arithmetic: no attention, no scoring,
no selection. Both the CPU oracle's tests and the GPU path's tests/bench take
their inputs from here, so the two sides always see bit-identical arrays.
"""
from .configs import WORKLOADS, Workload, workload  # noqa: F401
from .gen import (Inputs, IndexerInputs, make_inputs, make_projection_inputs, make_gates, make_indexer_inputs,  # noqa: F401
                  quantize_e4m3, checked_rows)
