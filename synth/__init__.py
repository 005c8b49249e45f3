"""Seeded synthetic inputs for vertical-slash sparse prefill.

This module only draws and shapes inputs (Gaussian Q/K/V, rotary position
embedding, planted vertical and periodic-diagonal structure).  It holds none of
the method's arithmetic, so both the CPU oracle and the GPU path can consume the
same tensors without sharing any code.
"""

from .gen import (WORKLOADS, DECODE_WORKLOADS, PACKED_WORKLOADS, DecodeWorkload, PackedWorkload, Workload,
                  make_decode_inputs, make_inputs, make_packed_inputs, small_workload, rope_tables)

__all__ = ["WORKLOADS", "DECODE_WORKLOADS", "PACKED_WORKLOADS", "Workload", "DecodeWorkload", "PackedWorkload",
           "make_inputs", "make_decode_inputs", "make_packed_inputs", "small_workload", "rope_tables"]
