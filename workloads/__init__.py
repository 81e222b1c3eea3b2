"""Seeded synthetic inputs shared by the parity tests, smoke() and bench.py."""
from . import synth  # noqa: F401
from .synth import (CONFIGS, PREFILL_CONFIGS, Workload, beam_fork, block_sweep,  # noqa: F401
                    gqa_suffix_lengths, independent, llama31_8b_prefill, prefill_chunks,
                    llama7b_mha, llama13b_beam, llama13b_long, llama31_8b_gqa,
                    normal_bits, shared_prefix, tiny)
