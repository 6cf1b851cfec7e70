"""Seeded synthetic workloads (recipes + input generator) shared by the oracle tests, the GPU
parity tests and the bench.  Holds none of the method's arithmetic."""
from .configs import ALL, BY_NAME, HEADLINE, Recipe  # noqa: F401
from .gen import Step, make_step, f32_to_bf16_bits, bf16_bits_to_f32, pack_k, pack_v  # noqa: F401
