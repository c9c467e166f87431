"""Seeded synthetic inputs for the tree-masked verify/expand attention path.

This package builds input arrays only: random queries/keys/values, parent
arrays, token ids and logits with planted accepted paths.  It holds none of
the method's arithmetic (no masks, no softmax, no argmax, no acceptance test,
no compaction); both the CPU oracle and the GPU path consume its output.
"""
from .workloads import (  # noqa: F401
    BF16_NAN_BITS,
    Case,
    bf16_bits_from_f32,
    config1_tiny,
    config2_chain,
    config3_tree,
    config4_expand,
    config5_paged,
    random_case,
)
