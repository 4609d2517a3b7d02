"""MI355X-native tree verification attention (LongSpec's Hybrid Tree Attention).

The compute path is ``libhta.so``: hand-written gfx950 HIP kernels behind the C ABI of
``include/hta.h``.  ``binding`` is its thin ctypes binding (same entry-point names);
``workloads`` draws the seeded synthetic inputs.  Around the attention, ``rope_tree`` encodes
the tree's positions and ``accept_commit`` accepts the greedy path and grows the KV cache.  The shared library is loaded on first
use and its absence is an error -- there is no CPU fallback.
"""
from .binding import (  # noqa: F401
    HtaError,
    accept_commit,
    accept_workspace_size,
    ancestor_masks,
    chunk_mass,
    cross_attention,
    dense_mask_shape,
    desc_for,
    hta_accept_commit,
    hta_ancestor_masks,
    hta_chunk_mass,
    hta_cross_attention,
    hta_dense_mask,
    hta_get_device_status,
    hta_merge,
    hta_prefix_partials,
    hta_rope_tree,
    hta_tree_partials,
    hta_verify,
    hta_verify_dense,
    hta_verify_noalloc,
    hta_window_commit,
    load,
    make_desc,
    new_workspace,
    partial_views,
    plan,
    prepare_accept_commit,
    prepare_chunk_mass,
    prepare_cross_attention,
    prepare_merge,
    prepare_mfma_peak_probe,
    prepare_prefix_partials,
    prepare_rope_tree,
    prepare_tree_partials,
    prepare_verify,
    rope_tree,
    status_str,
    verify,
    verify_dense,
    workspace_size,
)

__all__ = [
    "HtaError", "accept_commit", "accept_workspace_size", "ancestor_masks", "chunk_mass",
    "cross_attention", "dense_mask_shape", "desc_for", "hta_cross_attention",
    "hta_window_commit", "hta_accept_commit", "hta_ancestor_masks", "hta_chunk_mass",
    "hta_dense_mask", "hta_verify_dense", "verify_dense", "hta_get_device_status", "hta_merge",
    "hta_prefix_partials", "hta_rope_tree", "hta_tree_partials", "hta_verify", "hta_verify_noalloc", "load",
    "make_desc", "new_workspace", "partial_views", "plan", "prepare_accept_commit",
    "prepare_chunk_mass", "prepare_cross_attention", "prepare_merge", "prepare_mfma_peak_probe",
    "prepare_prefix_partials",
    "prepare_rope_tree", "prepare_tree_partials", "prepare_verify", "rope_tree", "status_str", "verify",
    "workspace_size",
]
