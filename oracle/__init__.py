"""CPU oracle for content-adaptive block-sparse video attention.

TEST INFRASTRUCTURE ONLY. The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only code allowed to import this
package. It shares no code, table or constant with the HIP library and never
calls it; the HIP library never imports it.

What it computes follows the NABLA technical summary (gist.science, paper
2507.13546, "Methodology" items 1-3) and, for the semantic-permutation
variant, the Sparse VideoGen2 technical summary (gist.science, paper
2505.18875, section 2 "Methodology" A-B). Arithmetic is numpy float64 on a
single thread unless a function states otherwise.

Parity status of each function is recorded in its docstring ("pinned by ...").
"""
from .nabla import (  # noqa: F401
    Grid,
    fractal_positions,
    valid_slots,
    block_coords,
    permute,
    unpermute,
    pool_blocks,
    block_logits,
    block_probs,
    cdf_cut,
    cdf_cut_details,
    topk_cut,
    topk_cut_details,
    sta_mask,
    sta_only_lists,
    build_block_mask,
    mask_to_lists,
    lists_to_mask,
    exempt_rows,
    bsa_forward,
    bsa_backward,
    dense_attention,
    masked_attention_bruteforce,
    layer,
)
from . import svg2  # noqa: F401,E402
