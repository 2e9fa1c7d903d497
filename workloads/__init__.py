"""Seeded synthetic inputs for paged-KV attention.

This package only draws numbers: context lengths, physical block assignments and
N(0, 1) tensors.  It holds none of the attention arithmetic, so both the CPU oracle
side and the HIP side of the tests can consume the same inputs without sharing any
computation.
"""
from .synth import (  # noqa: F401
    BLOCK_SIZE,
    CONFIG_NAMES,
    PagedBatch,
    make_config,
    make_batch,
    bf16_round_bits,
)
