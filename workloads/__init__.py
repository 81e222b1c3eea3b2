"""Seeded synthetic inputs shared by the parity tests, smoke() and bench.py."""
from . import synth  # noqa: F401
from .synth import (CONFIGS, Workload, beam_fork, block_sweep, gqa_suffix_lengths,  # noqa: F401
                    independent,
                    llama7b_mha, llama13b_beam, llama13b_long, llama31_8b_gqa,
                    normal_bits, shared_prefix, tiny)
