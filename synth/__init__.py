"""Seeded synthetic inputs (shapes and planted structure) shared by the oracle tests,
the GPU parity tests and the benchmark.  Holds none of the attention method's arithmetic."""
from .configs import Config, CONFIGS, BY_INDEX, C0, C1, C2, C3, C4, M1, M2, M3, M4, M5, M6, with_  # noqa: F401
from .workload import Workload, chunk_prompt_sequence, chunk_prompts, layer_arrays, round_bf16, stack_host_pages, to_bf16_bits  # noqa: F401
