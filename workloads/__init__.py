"""Seeded synthetic inputs for the MLA tree-verify attention.

This module is shared by the CPU oracle tests, the HIP parity tests and the
benchmark. It draws draft trees, builds the tree visibility masks, samples KV
pool slots and draws bf16 values. It holds none of the attention arithmetic
(no scores, no softmax, no weighted sums), so neither side can borrow the
other's mathematics through it.

Shapes and the visibility rule follow the workloads of the pages
"From Capture Safety to MoE Ceiling" (section "The Architecture of Capture
Safety": prefix slots in kv_indices, draft slots in out_cache_loc, raw
custom_mask + mask_indptr) and "The Custom sm_120 Verify Kernel" (section
"The Debugging Gauntlet", bug 2: mask rows are prefix + q_len wide).
"""
from .gen import (  # noqa: F401
    BF16_NAN,
    CONFIGS,
    Inputs,
    Workload,
    bf16_from_f32,
    bf16_to_f32,
    chain_tree,
    compact_inputs,
    full_pool,
    make_inputs,
    make_custom,
    random_tree,
    tree_mask,
)
