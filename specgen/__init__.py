"""Seeded synthetic inputs for the branch-parallel scoring path.

This package is the only code shared by the CPU oracle and the HIP path. It
draws tree structures, Q/K/V tensors, logit rows, GDN replay inputs and the
indexer queries and keys of sparse attention from
counter-addressed NumPy PCG64 streams (hidden states
and output heads too) and rounds them to bfloat16 where a
workload asks for it.
It holds none of the method's arithmetic (no packing, attention or loss).
"""
from .configs import CONFIGS, Config, get_config, small_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gen_gdn,
    gen_gdn_states,
    gen_head,
    gen_head_draft_rows,
    gen_logits,
    gen_logit_rows,
    gen_qkv,
    gen_qsa_index,
    gen_structure,
)
