"""Seeded, synthetic inputs for the PTX-subset SIMT simulator.

This package produces *inputs only*: PTX program text, initial simulated-memory
images, parameter blocks and launch shapes.  It holds none of the simulator's
arithmetic, so both the GPU path's tests and the CPU oracle can consume it.
"""
from .configs import (Workload, vector_add, strided_gather, ffma_probe, bank_probe, random_stress,
                      pack_params, LAT_DEFAULT_NOTE)
from .randprog import random_program

__all__ = ["Workload", "vector_add", "strided_gather", "ffma_probe", "bank_probe", "random_stress",
           "random_program", "pack_params", "LAT_DEFAULT_NOTE"]
