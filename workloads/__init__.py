"""Seeded synthetic inputs (sector structures, layouts and values) shared by the
oracle tests, the GPU parity tests and the benchmark.  No contraction arithmetic."""
from .model import Index, Operand, Contraction, Problem, Stage, Chain, bf16_round, bf16_bits  # noqa: F401
from . import configs  # noqa: F401
