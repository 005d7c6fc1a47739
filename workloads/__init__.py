"""Seeded synthetic inputs for document-masked varlen attention.

This package is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``load_balance_amd/``).  It draws document lengths and q/k/v values
and rounds them to bfloat16; it holds none of the attention arithmetic, none
of the masking rules and none of the sharding rules.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    lognormal_lengths,
    cu_from_lengths,
    tiny_pack,
    longtail_pack,
    pair_packs,
    zigzag_pack_lengths,
    zigzag_chunk_values,
    shared_question_packs,
    values,
)
