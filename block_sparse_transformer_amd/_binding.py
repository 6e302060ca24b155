"""ctypes marshalling for libbsattn.so (see include/bsattn.h for the contract)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSATTN_LIBRARY names another build of the library (e.g. libbsattn_debug.so)
_LIB_PATH = os.environ.get("BSATTN_LIBRARY") or os.path.join(_HERE, "libbsattn.so")
_lib = None

BSATTN_F32 = 0
BSATTN_BF16 = 1

_c_int = ctypes.c_int32
_c_vp = ctypes.c_void_p
_c_i32p = ctypes.POINTER(ctypes.c_int32)


class BsattnError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {bsattn_status_string(status)}: {bsattn_last_error()}")


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libbsattn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m block_sparse_transformer_amd.build` "
            "(or __graft_entry__.build()). There is no CPU fallback.")
    L = ctypes.CDLL(_LIB_PATH)
    L.bsattn_make_layout.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_i32p, _c_int, _c_int,
                                     ctypes.c_uint64, ctypes.POINTER(_c_vp)]
    L.bsattn_make_band_layout.argtypes = [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_c_vp)]
    L.bsattn_make_token_layout.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_uint64,
                                           ctypes.POINTER(_c_vp)]
    L.bsattn_make_adaptive_layout.argtypes = [_c_int, _c_int, _c_int, ctypes.POINTER(_c_vp)]
    L.bsattn_adaptive_select.argtypes = [_c_vp, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                         ctypes.c_size_t, _c_vp]
    L.bsattn_make_topr_layout.argtypes = [_c_int, _c_int, _c_int, ctypes.POINTER(_c_vp)]
    L.bsattn_topr_select.argtypes = [_c_vp, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                     ctypes.c_size_t, _c_vp]
    L.bsattn_layout_token_links.argtypes = [_c_vp, ctypes.POINTER(_c_i32p), ctypes.POINTER(_c_int),
                                            ctypes.POINTER(_c_i32p), ctypes.POINTER(_c_int)]
    L.bsattn_layout_csr.argtypes = [_c_vp, ctypes.POINTER(_c_i32p), ctypes.POINTER(_c_i32p),
                                    ctypes.POINTER(_c_int), ctypes.POINTER(ctypes.c_int64)]
    L.bsattn_layout_tile_masks.argtypes = [_c_vp, ctypes.POINTER(ctypes.POINTER(ctypes.c_uint8)),
                                           ctypes.POINTER(ctypes.c_int64)]
    L.bsattn_layout_upload.argtypes = [_c_vp, _c_vp]
    L.bsattn_layout_build_device.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp]
    L.bsattn_layout_destroy.argtypes = [_c_vp]
    L.bsattn_layout_destroy.restype = None
    L.bsattn_workspace_size.argtypes = [_c_vp, _c_int, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bsattn_forward.argtypes = [_c_vp, ctypes.c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                 _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_vp, ctypes.c_size_t, _c_vp]
    L.bsattn_route_workspace_size.argtypes = [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bsattn_route_topk.argtypes = [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp,
                                    ctypes.c_size_t, _c_vp]
    L.bsattn_forward_routed.argtypes = [_c_vp, ctypes.c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp,
                                        _c_vp, _c_vp, _c_int, _c_vp, _c_vp, ctypes.c_float, _c_vp,
                                        ctypes.c_size_t, _c_vp]
    L.bsattn_backward_workspace_size.argtypes = [_c_vp, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bsattn_backward.argtypes = [_c_vp, ctypes.c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                  _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_vp,
                                  ctypes.c_size_t, _c_vp]
    L.bsattn_backward_routed_workspace_size.argtypes = [_c_vp, _c_int, _c_int, _c_int,
                                                        ctypes.POINTER(ctypes.c_size_t)]
    L.bsattn_backward_routed.argtypes = [_c_vp, ctypes.c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                         _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_vp, ctypes.c_float,
                                         _c_vp, ctypes.c_size_t, _c_vp]
    L.bsattn_layer_workspace_size.argtypes = [_c_vp, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.bsattn_layer_forward.argtypes = [_c_vp, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                       _c_vp, _c_vp, ctypes.c_float, _c_vp, ctypes.c_size_t, _c_vp]
    L.bsattn_candidate_positions.argtypes = [_c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp]
    L.bsattn_candidate_forward.argtypes = [ctypes.c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                           _c_vp, _c_int, _c_int, ctypes.c_float, _c_vp, _c_vp, _c_vp, _c_vp]
    L.bsattn_set_profile_events.argtypes = [_c_vp, _c_vp]
    L.bsattn_prepare.argtypes = [_c_vp, _c_int, _c_int, _c_int, _c_int, _c_vp]
    L.bsattn_forward_noalloc.argtypes = [_c_vp, ctypes.c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp,
                                         _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, _c_vp]
    L.bsattn_status_string.argtypes = [ctypes.c_int]
    L.bsattn_status_string.restype = ctypes.c_char_p
    L.bsattn_last_error.argtypes = []
    L.bsattn_last_error.restype = ctypes.c_char_p
    for name in ("bsattn_make_layout", "bsattn_make_band_layout", "bsattn_make_token_layout",
                 "bsattn_make_adaptive_layout", "bsattn_adaptive_select",
                 "bsattn_make_topr_layout", "bsattn_topr_select",
                 "bsattn_layout_token_links", "bsattn_layout_csr",
                 "bsattn_layout_tile_masks", "bsattn_layout_upload",
                 "bsattn_layout_build_device", "bsattn_workspace_size", "bsattn_forward",
                 "bsattn_route_topk", "bsattn_route_workspace_size", "bsattn_forward_routed",
                 "bsattn_set_profile_events",
                 "bsattn_prepare", "bsattn_forward_noalloc", "bsattn_backward_routed_workspace_size",
                 "bsattn_backward_routed", "bsattn_candidate_positions", "bsattn_candidate_forward"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def bsattn_status_string(status: int) -> str:
    return lib().bsattn_status_string(int(status)).decode()


def bsattn_last_error() -> str:
    return lib().bsattn_last_error().decode()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise BsattnError(func, status)


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Layout:
    """Owner of a ``bsattn_layout*``; freed on destroy() or garbage collection."""

    def __init__(self, handle: int, num_heads: int, seq_len: int, band_tokens: Optional[int] = None):
        self._h = handle
        self.num_heads = num_heads
        self.seq_len = seq_len
        self.band_tokens = band_tokens

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("layout has been destroyed")
        return self._h

    def destroy(self) -> None:
        if self._h:
            lib().bsattn_layout_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def bsattn_make_layout(num_heads: int, seq_len: int, block: int, window_blocks: int,
                       global_blocks: Sequence[int], random_blocks: int, seed: int) -> Layout:
    g = (ctypes.c_int32 * max(1, len(global_blocks)))(*global_blocks)
    out = _c_vp()
    _check("bsattn_make_layout", lib().bsattn_make_layout(
        num_heads, seq_len, block, window_blocks, g if len(global_blocks) else None, len(global_blocks),
        random_blocks, ctypes.c_uint64(seed & ((1 << 64) - 1)), ctypes.byref(out)))
    return Layout(out.value, num_heads, seq_len)


def bsattn_make_band_layout(num_heads: int, seq_len: int, block: int, band_tokens: int) -> Layout:
    out = _c_vp()
    _check("bsattn_make_band_layout", lib().bsattn_make_band_layout(num_heads, seq_len, block, band_tokens,
                                                                    ctypes.byref(out)))
    return Layout(out.value, num_heads, seq_len, band_tokens=band_tokens)


def bsattn_make_token_layout(num_heads: int, seq_len: int, band_tokens: int, num_global: int,
                             random_tokens: int, seed: int) -> Layout:
    out = _c_vp()
    _check("bsattn_make_token_layout", lib().bsattn_make_token_layout(
        num_heads, seq_len, band_tokens, num_global, random_tokens, ctypes.c_uint64(seed & ((1 << 64) - 1)),
        ctypes.byref(out)))
    return Layout(out.value, num_heads, seq_len, band_tokens=band_tokens)


def bsattn_make_adaptive_layout(num_heads: int, seq_len: int, keep_blocks: int) -> Layout:
    out = _c_vp()
    _check("bsattn_make_adaptive_layout", lib().bsattn_make_adaptive_layout(num_heads, seq_len, keep_blocks,
                                                                            ctypes.byref(out)))
    lay = Layout(out.value, num_heads, seq_len)
    lay.keep_blocks = keep_blocks
    return lay


def bsattn_adaptive_select(layout: Layout, q, k, workspace=None, stream=None):
    """The kept key blocks [B, H, L/64, keep] (device int32) of an adaptive layout for q, k."""
    import torch
    B, H, L, D = q.shape
    cols = torch.empty((B, H, L // 64, layout.keep_blocks), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = _workspace(layout, q)
    _check("bsattn_adaptive_select", lib().bsattn_adaptive_select(
        layout.handle, B, H, L, D, q.data_ptr(), k.data_ptr(), cols.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return cols


def bsattn_make_topr_layout(num_heads: int, seq_len: int, keep_tokens: int) -> Layout:
    out = _c_vp()
    _check("bsattn_make_topr_layout", lib().bsattn_make_topr_layout(num_heads, seq_len, keep_tokens,
                                                                    ctypes.byref(out)))
    lay = Layout(out.value, num_heads, seq_len)
    lay.keep_tokens = keep_tokens
    return lay


def bsattn_topr_select(layout: Layout, q, k, workspace=None, stream=None):
    """The kept-key words [B, H, L, L/64] (device int64; bit b of word j: key 64 j + b) of a
    top-keep layout for q, k."""
    import torch
    B, H, L, D = q.shape
    bits = torch.empty((B, H, L, L // 64), dtype=torch.int64, device=q.device)
    if workspace is None:
        workspace = _workspace(layout, q)
    _check("bsattn_topr_select", lib().bsattn_topr_select(
        layout.handle, B, H, L, D, q.data_ptr(), k.data_ptr(), bits.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return bits


def bsattn_candidate_positions(x, w, bias, positions=None, stream=None):
    """Candidate positions [B, L, k] (device int32) of the hidden states x (bf16 [B, L, C]);
    w fp32 [3, C, k] (tap-major Conv1d weight), bias fp32 [k]."""
    import torch
    B, L, C = x.shape
    k = w.shape[2]
    if x.dtype != torch.bfloat16 or w.dtype != torch.float32 or bias.dtype != torch.float32:
        raise ValueError("x must be bf16, w and bias fp32")
    if tuple(w.shape) != (3, C, k) or tuple(bias.shape) != (k,) or not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("w must be a contiguous [3, C, k] tensor and bias [k]")
    if positions is None:
        positions = torch.empty((B, L, k), dtype=torch.int32, device=x.device)
    _check("bsattn_candidate_positions", lib().bsattn_candidate_positions(
        x.data_ptr(), w.data_ptr(), bias.data_ptr(), B, L, C, k, positions.data_ptr(), _stream_handle(stream)))
    return positions


def bsattn_candidate_forward(q, k, v, positions, keep: int, scale: Optional[float] = None, out=None, lse=None,
                             kept=None, stream=None):
    """Attention of every query over its `keep` best candidates; returns (out, lse)."""
    import torch
    _check_qkv(q, k, v, q if out is None else out)
    B, H, L, D = q.shape
    n_cand = positions.shape[-1]
    if positions.dtype != torch.int32 or tuple(positions.shape) != (B, L, n_cand) or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int32 [B, L, k] tensor")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    _check("bsattn_candidate_forward", lib().bsattn_candidate_forward(
        _dtype_code(q), B, H, L, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), positions.data_ptr(), n_cand,
        int(keep), scale, out.data_ptr(), lse.data_ptr(), None if kept is None else kept.data_ptr(),
        _stream_handle(stream)))
    return out, lse


def bsattn_layout_token_links(layout: Layout) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of a token layout's global tokens [n] and random tokens [H, L, r] (-1 padded)."""
    g, lk = _c_i32p(), _c_i32p()
    ng, r = _c_int(), _c_int()
    _check("bsattn_layout_token_links", lib().bsattn_layout_token_links(layout.handle, ctypes.byref(g),
                                                                        ctypes.byref(ng), ctypes.byref(lk),
                                                                        ctypes.byref(r)))
    gt = np.ctypeslib.as_array(g, shape=(ng.value,)).copy() if ng.value else np.zeros(0, np.int32)
    shape = (layout.num_heads, layout.seq_len, r.value)
    links = (np.ctypeslib.as_array(lk, shape=shape).copy() if r.value else np.zeros(shape, np.int32))
    return gt, links


def bsattn_layout_csr(layout: Layout) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the host CSR arrays (row_ptr [rows+1], col_idx [nnz]) as int32 numpy."""
    rp, ci = _c_i32p(), _c_i32p()
    nrows, nnz = _c_int(), ctypes.c_int64()
    _check("bsattn_layout_csr", lib().bsattn_layout_csr(layout.handle, ctypes.byref(rp), ctypes.byref(ci),
                                                        ctypes.byref(nrows), ctypes.byref(nnz)))
    row_ptr = np.ctypeslib.as_array(rp, shape=(nrows.value + 1,)).copy()
    col = np.ctypeslib.as_array(ci, shape=(max(1, nnz.value),))[: nnz.value].copy()
    return row_ptr, col


def bsattn_layout_tile_masks(layout: Layout) -> Optional[np.ndarray]:
    """Copy of the quarter masks (uint8 [nnz], bit 2a + b: query half a sees key
    half b) of a layout of 32-token blocks; None for other layouts."""
    p = ctypes.POINTER(ctypes.c_uint8)()
    n = ctypes.c_int64()
    _check("bsattn_layout_tile_masks", lib().bsattn_layout_tile_masks(layout.handle, ctypes.byref(p),
                                                                      ctypes.byref(n)))
    if not p or n.value == 0:
        return None
    return np.ctypeslib.as_array(p, shape=(n.value,)).copy()


def bsattn_layout_upload(layout: Layout, stream=None) -> None:
    _check("bsattn_layout_upload", lib().bsattn_layout_upload(layout.handle, _stream_handle(stream)))


def bsattn_prepare(layout: Layout, batch: int, head_dim: int, num_routed: int = 0, backward: bool = False,
                   stream=None) -> None:
    """Build and upload the schedule of one call shape ahead of time (see bsattn.h)."""
    _check("bsattn_prepare", lib().bsattn_prepare(layout.handle, batch, head_dim, num_routed, int(bool(backward)),
                                                  _stream_handle(stream)))


def bsattn_layout_build_device(layout: Layout, row_ptr_dev, col_idx_dev, tile_masks_dev=None,
                               stream=None) -> None:
    """The layout rebuilt on the device into caller tensors (tile_masks_dev: uint8 [nnz],
    needed for layouts of 32-token blocks)."""
    _check("bsattn_layout_build_device", lib().bsattn_layout_build_device(
        layout.handle, _ptr(row_ptr_dev), _ptr(col_idx_dev), _ptr(tile_masks_dev), _stream_handle(stream)))


def bsattn_layout_destroy(layout: Layout) -> None:
    layout.destroy()


def bsattn_workspace_size(layout: Layout, batch: int, head_dim: int, num_routed: int = 0) -> int:
    n = ctypes.c_size_t()
    _check("bsattn_workspace_size", lib().bsattn_workspace_size(layout.handle, batch, head_dim, num_routed,
                                                                ctypes.byref(n)))
    return n.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BSATTN_BF16
    if t.dtype == torch.float32:
        return BSATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_qkv(q, k, v, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4 or tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"{name} must have the shape of q {tuple(q.shape)}")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q's dtype and device")


def bsattn_forward(layout: Layout, q, k, v, out, lse, key_valid_len=None, scale: Optional[float] = None,
                   workspace=None, stream=None) -> None:
    """Enqueue the forward pass; all tensors are caller-allocated device tensors."""
    import torch
    _check_qkv(q, k, v, out)
    B, H, L, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, L] tensor")
    if key_valid_len is not None and (key_valid_len.dtype != torch.int32 or key_valid_len.numel() != B):
        raise ValueError("key_valid_len must be int32 [B]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bsattn_forward", lib().bsattn_forward(
        layout.handle, _dtype_code(q), B, H, L, D, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
        _ptr(key_valid_len), scale, _ptr(workspace), wbytes, _stream_handle(stream)))


def bsattn_forward_noalloc(layout: Layout, q, k, v, out, lse, key_valid_len=None, scale: Optional[float] = None,
                           stream=None) -> None:
    """Enqueue the forward with the library's own device scratch as workspace (no allocation;
    the shape must have been prepared with :func:`bsattn_prepare`)."""
    import torch
    _check_qkv(q, k, v, out)
    B, H, L, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, L] tensor")
    if key_valid_len is not None and (key_valid_len.dtype != torch.int32 or key_valid_len.numel() != B):
        raise ValueError("key_valid_len must be int32 [B]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    _check("bsattn_forward_noalloc", lib().bsattn_forward_noalloc(
        layout.handle, _dtype_code(q), B, H, L, D, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
        _ptr(key_valid_len), scale, _stream_handle(stream)))


def bsattn_route_workspace_size(batch: int, num_heads: int, seq_len: int, k: int) -> int:
    n = ctypes.c_size_t()
    _check("bsattn_route_workspace_size", lib().bsattn_route_workspace_size(batch, num_heads, seq_len, k,
                                                                            ctypes.byref(n)))
    return n.value


def bsattn_route_topk(q, w, k: int, routed_rows, workspace=None, stream=None) -> None:
    """Router top-k into routed_rows; a workspace of bsattn_route_workspace_size bytes
    (uint8, on q's device) is allocated here when none is given."""
    import torch
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be a contiguous bf16 [B, H, L, D] tensor")
    B, H, L, D = q.shape
    if w.dtype != torch.float32 or w.numel() != D:
        raise ValueError("w must be fp32 [D]")
    if routed_rows.dtype != torch.int32 or tuple(routed_rows.shape) != (B, H, k):
        raise ValueError("routed_rows must be int32 [B, H, k]")
    need = bsattn_route_workspace_size(B, H, L, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check("bsattn_route_topk", lib().bsattn_route_topk(_ptr(q), _ptr(w), B, H, L, D, k, _ptr(routed_rows),
                                                        _ptr(workspace), nbytes, _stream_handle(stream)))


def bsattn_forward_routed(band_layout: Layout, q, k, v, routed_rows, out, lse, scale: Optional[float] = None,
                          workspace=None, stream=None) -> None:
    import torch
    _check_qkv(q, k, v, out)
    B, H, L, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, L] tensor")
    if routed_rows.dtype != torch.int32 or routed_rows.dim() != 3 or tuple(routed_rows.shape[:2]) != (B, H):
        raise ValueError("routed_rows must be int32 [B, H, k]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bsattn_forward_routed", lib().bsattn_forward_routed(
        band_layout.handle, _dtype_code(q), B, H, L, D, _ptr(q), _ptr(k), _ptr(v), _ptr(routed_rows),
        int(routed_rows.shape[2]), _ptr(out), _ptr(lse), scale, _ptr(workspace), wbytes,
        _stream_handle(stream)))


def bsattn_backward_workspace_size(layout: Layout, batch: int, head_dim: int) -> int:
    n = ctypes.c_size_t()
    _check("bsattn_backward_workspace_size",
           lib().bsattn_backward_workspace_size(layout.handle, batch, head_dim, ctypes.byref(n)))
    return n.value


def bsattn_backward(layout: Layout, q, k, v, out, lse, dout, dq, dk, dv, key_valid_len=None,
                    scale: Optional[float] = None, workspace=None, stream=None) -> None:
    """Enqueue the backward pass; all tensors are caller-allocated device tensors."""
    import torch
    _check_qkv(q, k, v, out)
    _check_qkv(q, dout, dq, dk)
    _check_qkv(q, dv, dv, dv)
    B, H, L, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, L] tensor")
    if key_valid_len is not None and (key_valid_len.dtype != torch.int32 or key_valid_len.numel() != B):
        raise ValueError("key_valid_len must be int32 [B]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bsattn_backward", lib().bsattn_backward(
        layout.handle, _dtype_code(q), B, H, L, D, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(key_valid_len), scale, _ptr(workspace), wbytes,
        _stream_handle(stream)))


def bsattn_backward_routed_workspace_size(layout: Layout, batch: int, head_dim: int, num_routed: int) -> int:
    n = ctypes.c_size_t()
    _check("bsattn_backward_routed_workspace_size", lib().bsattn_backward_routed_workspace_size(
        layout.handle, batch, head_dim, num_routed, ctypes.byref(n)))
    return n.value


def bsattn_backward_routed(band_layout: Layout, q, k, v, out, lse, dout, routed_rows, dq, dk, dv,
                           scale: Optional[float] = None, workspace=None, stream=None) -> None:
    """Enqueue the routed-query backward; all tensors are caller-allocated device tensors."""
    import torch
    _check_qkv(q, k, v, out)
    _check_qkv(q, dout, dq, dk)
    _check_qkv(q, dv, dv, dv)
    B, H, L, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, L] tensor")
    if routed_rows.dtype != torch.int32 or routed_rows.dim() != 3 or tuple(routed_rows.shape[:2]) != (B, H) \
            or not routed_rows.is_contiguous():
        raise ValueError("routed_rows must be a contiguous int32 [B, H, k] tensor")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bsattn_backward_routed", lib().bsattn_backward_routed(
        band_layout.handle, _dtype_code(q), B, H, L, D, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
        _ptr(dout), _ptr(routed_rows), int(routed_rows.shape[2]), _ptr(dq), _ptr(dk), _ptr(dv), scale,
        _ptr(workspace), wbytes, _stream_handle(stream)))


def bsattn_layer_workspace_size(layout: Layout, batch: int, head_dim: int) -> int:
    n = ctypes.c_size_t()
    _check("bsattn_layer_workspace_size",
           lib().bsattn_layer_workspace_size(layout.handle, batch, head_dim, ctypes.byref(n)))
    return n.value


def bsattn_layer_forward(layout: Layout, x, w_qkv, b_qkv, w_proj, b_proj, out, num_heads: int,
                         key_valid_len=None, scale: Optional[float] = None, workspace=None, stream=None) -> None:
    """Enqueue the attention layer; all tensors are caller-allocated bf16 device tensors."""
    import torch
    B, L, C = x.shape
    D = C // num_heads
    shapes = {"x": (x, (B, L, C)), "w_qkv": (w_qkv, (3 * C, C)), "b_qkv": (b_qkv, (3 * C,)),
              "w_proj": (w_proj, (C, C)), "b_proj": (b_proj, (C,)), "out": (out, (B, L, C))}
    for name, (t, shape) in shapes.items():
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shape}")
    if key_valid_len is not None and (key_valid_len.dtype != torch.int32 or key_valid_len.numel() != B):
        raise ValueError("key_valid_len must be int32 [B]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bsattn_layer_forward", lib().bsattn_layer_forward(
        layout.handle, B, num_heads, L, D, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_proj), _ptr(b_proj),
        _ptr(out), _ptr(key_valid_len), scale, _ptr(workspace), wbytes, _stream_handle(stream)))


def layer_forward(x, w_qkv, b_qkv, w_proj, b_proj, layout: Layout, num_heads: int, key_valid_len=None,
                  scale: Optional[float] = None, workspace=None):
    """Allocate out and workspace with torch and run :func:`bsattn_layer_forward`."""
    import torch
    out = torch.empty_like(x)
    if workspace is None:
        n = bsattn_layer_workspace_size(layout, x.shape[0], x.shape[2] // num_heads)
        workspace = torch.empty((n + 255) // 4, dtype=torch.float32, device=x.device)
    bsattn_layer_forward(layout, x, w_qkv, b_qkv, w_proj, b_proj, out, num_heads, key_valid_len, scale, workspace)
    return out


def bsattn_set_profile_events(before: Optional[int], after: Optional[int]) -> None:
    _check("bsattn_set_profile_events", lib().bsattn_set_profile_events(before, after))


def _workspace(layout: Layout, q, num_routed: int = 0):
    import torch
    n = bsattn_workspace_size(layout, q.shape[0], q.shape[3], num_routed)
    if n == 0:
        return None
    return torch.empty((n + 255) // 4, dtype=torch.float32, device=q.device)


def forward(q, k, v, layout: Layout, key_valid_len=None, scale: Optional[float] = None, workspace=None):
    """Allocate (out, lse) with torch and run :func:`bsattn_forward` on the current stream."""
    import torch
    B, H, L, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(layout, q)
    bsattn_forward(layout, q, k, v, out, lse, key_valid_len, scale, workspace)
    return out, lse


def backward(q, k, v, out, lse, dout, layout: Layout, key_valid_len=None, scale: Optional[float] = None,
             workspace=None):
    """Allocate (dq, dk, dv) and workspace with torch and run :func:`bsattn_backward`."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if workspace is None:
        n = bsattn_backward_workspace_size(layout, q.shape[0], q.shape[3])
        workspace = torch.empty((n + 255) // 4, dtype=torch.float32, device=q.device)
    bsattn_backward(layout, q, k, v, out, lse, dout, dq, dk, dv, key_valid_len, scale, workspace)
    return dq, dk, dv


def backward_routed(q, k, v, out, lse, dout, band_layout: Layout, routed_rows, scale: Optional[float] = None,
                    workspace=None):
    """Allocate (dq, dk, dv) and workspace with torch and run :func:`bsattn_backward_routed`."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if workspace is None:
        n = bsattn_backward_routed_workspace_size(band_layout, q.shape[0], q.shape[3], int(routed_rows.shape[2]))
        workspace = torch.empty((n + 255) // 4, dtype=torch.float32, device=q.device)
    bsattn_backward_routed(band_layout, q, k, v, out, lse, dout, routed_rows, dq, dk, dv, scale, workspace)
    return dq, dk, dv


def forward_routed(q, k, v, band_layout: Layout, routed_rows, scale: Optional[float] = None, workspace=None):
    import torch
    B, H, L, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(band_layout, q, int(routed_rows.shape[2]))
    bsattn_forward_routed(band_layout, q, k, v, routed_rows, out, lse, scale, workspace)
    return out, lse


# hipEventDisableSystemFence: the event only takes a timestamp; recording it does
# not write back and invalidate the caches (HIP documents the flag for events used
# only to measure time).  Readers synchronise the device before reading the times.
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Raw hipEvent_t pairs from the HIP runtime, for timing one kernel on a given stream.

    The events are timing-only (no system-scope fence when recorded), so that
    recording them between kernels does not add cache writebacks to the timed
    work; synchronise the device before calling elapsed_ms."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_c_vp), ctypes.c_uint]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _c_vp, _c_vp]
        self._hip.hipEventSynchronize.argtypes = [_c_vp]
        self._hip.hipEventDestroy.argtypes = [_c_vp]
        self.before, self.after = [], []
        for _ in range(n):
            for lst in (self.before, self.after):
                e = _c_vp()
                if self._hip.hipEventCreateWithFlags(ctypes.byref(e), _HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                lst.append(e.value)

    def elapsed_ms(self, i: int) -> float:
        ms = ctypes.c_float()
        if self._hip.hipEventSynchronize(self.after[i]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.before[i], self.after[i]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self) -> None:
        for e in self.before + self.after:
            self._hip.hipEventDestroy(e)
        self.before, self.after = [], []
