"""block_sparse_transformer_amd -- block-sparse attention forward and backward on AMD MI355X (gfx950).

A thin ctypes binding of ``libbsattn.so`` (declared in ``include/bsattn.h``).
Every function here only marshals arguments: tensors become device pointers,
the current torch stream becomes the ``hipStream_t``.  All computation runs in
the HIP kernels of the library; there is no CPU fallback, and every function
raises if the library has not been built.

Functions carry the C names (``bsattn_make_layout``, ``bsattn_forward``, ...)
plus conveniences, :func:`forward`, :func:`forward_routed`, :func:`backward`
and :func:`layer_forward`, that allocate outputs and workspace with torch.
"""
from ._binding import (  # noqa: F401
    BsattnError,
    Layout,
    backward,
    backward_routed,
    bsattn_adaptive_select,
    bsattn_backward,
    bsattn_backward_routed,
    bsattn_backward_routed_workspace_size,
    bsattn_backward_workspace_size,
    bsattn_candidate_forward,
    bsattn_candidate_positions,
    bsattn_forward,
    bsattn_forward_noalloc,
    bsattn_forward_routed,
    bsattn_last_error,
    bsattn_layer_forward,
    bsattn_layer_workspace_size,
    bsattn_layout_build_device,
    bsattn_layout_csr,
    bsattn_layout_destroy,
    bsattn_layout_tile_masks,
    bsattn_layout_token_links,
    bsattn_layout_upload,
    bsattn_make_band_layout,
    bsattn_make_adaptive_layout,
    bsattn_make_layout,
    bsattn_make_token_layout,
    bsattn_make_topr_layout,
    bsattn_prepare,
    bsattn_route_topk,
    bsattn_route_workspace_size,
    bsattn_set_profile_events,
    bsattn_status_string,
    bsattn_topr_select,
    bsattn_workspace_size,
    forward,
    forward_routed,
    layer_forward,
    lib,
    library_path,
    HipEvents,
)
