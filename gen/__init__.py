"""Seeded synthetic input generators shared by the oracle tests, the GPU tests and the benchmark.

This package draws random tensors and packs them into the storage formats the library consumes
(fp32, or bf16 bit patterns). It holds none of the scan's arithmetic: no apply, no update, no
prefix accumulation, no TTT-Linear step and no routing decision.
"""
from .synth import *  # noqa: F401,F403
