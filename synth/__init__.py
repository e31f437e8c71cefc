"""Seeded synthetic workloads (inputs only; no compression arithmetic)."""
from .gen import (WORKLOADS, WORKLOAD_ORDER, Workload, layer_tensors, unit_inputs, seq_lengths,
                  bf16_bits, noise, stream_key)

__all__ = ["WORKLOADS", "WORKLOAD_ORDER", "Workload", "layer_tensors", "unit_inputs",
           "seq_lengths", "bf16_bits", "noise", "stream_key"]
