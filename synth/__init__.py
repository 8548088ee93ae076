"""Seeded synthetic inputs shared by the HIP path's harness and the CPU oracle (random draws only)."""
from .workloads import (DECODING, PREFILLING, WAITING, LayerSpec, Request, Workload, make_workload,
                        ring_pages_needed, round_to_bf16, bf16_bits)

__all__ = ["DECODING", "PREFILLING", "WAITING", "LayerSpec", "Request", "Workload", "make_workload",
           "ring_pages_needed", "round_to_bf16", "bf16_bits"]
