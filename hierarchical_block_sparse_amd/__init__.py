"""Pyramid top-K block selection + block-sparse causal attention for AMD MI355X.

The compute path is libpyr.so (HIP kernels for gfx950 behind the C ABI of
include/pyr.h); this package is its thin ctypes binding.  Importing the package
does not load the library; the first call does, and fails loudly if the library
is missing.
"""

from ._binding import (  # noqa: F401
    PYR_BF16, PYR_F32, Problem, PyrError, alloc_bwd_workspace, alloc_pyramid, alloc_sel,
    alloc_trace, alloc_workspace, backward, declared_functions, forward, forward_packed, lib,
    problem_for, problem_for_packed,
    pyr_abi_version, pyr_append_pyramid, pyr_attn_bwd_workspace_bytes, pyr_attn_workspace_bytes,
    pyr_block_sparse_attn, pyr_block_sparse_attn_bwd, pyr_block_sparse_attn_noalloc,
    pyr_build_pyramid, pyr_level_offset,
    pyr_num_levels, pyr_num_query_blocks, pyr_pyramid_nodes, pyr_pyramid_planes,
    pyr_budgets_from_entropy, pyr_select_attn, pyr_select_topk, pyr_select_topk_budgets,
    pyramid_shape,
)
