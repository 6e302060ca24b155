"""The C ABI loads, exports every declared symbol, and rejects bad arguments
before touching the GPU (CPU only: no compute call is made here)."""
import ctypes
import os
import re

import pytest

import block_sparse_transformer_amd as bs
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bsattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsattn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert names == sorted([
        "bsattn_make_layout", "bsattn_make_band_layout", "bsattn_layout_csr", "bsattn_layout_upload",
        "bsattn_layout_tile_masks", "bsattn_layout_build_device", "bsattn_make_token_layout",
        "bsattn_layout_token_links", "bsattn_make_adaptive_layout", "bsattn_adaptive_select",
        "bsattn_make_topr_layout", "bsattn_topr_select", "bsattn_candidate_positions", "bsattn_candidate_forward",
        "bsattn_layout_destroy", "bsattn_workspace_size",
        "bsattn_forward", "bsattn_backward_workspace_size", "bsattn_backward",
        "bsattn_layer_workspace_size", "bsattn_layer_forward",
        "bsattn_route_topk", "bsattn_route_workspace_size", "bsattn_backward_routed", "bsattn_backward_routed_workspace_size", "bsattn_forward_routed", "bsattn_set_profile_events", "bsattn_status_string",
        "bsattn_last_error", "bsattn_prepare", "bsattn_forward_noalloc"])
    lib = bs.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_debug_build_exports_the_same_symbols():
    """libbsattn_debug.so (-DBSATTN_DEBUG, built by __graft_entry__.build()) is the same C ABI."""
    path = os.path.join(os.path.dirname(bs.library_path()), "libbsattn_debug.so")
    assert os.path.exists(path), f"{path} is missing: run __graft_entry__.build()"
    dbg = ctypes.CDLL(path)
    for n in _declared():
        assert hasattr(dbg, n), n


def test_status_strings_and_last_error():
    for code in range(6):
        assert bs.bsattn_status_string(code)
    assert bs.bsattn_status_string(99) == "unknown status"
    assert isinstance(bs.bsattn_last_error(), str)


@pytest.mark.parametrize("kw,code", [
    (dict(block=16), 2),
    (dict(block=256), 2),
    (dict(block=32, seq_len=32 * 33), 1),
    (dict(seq_len=100), 1),
    (dict(window_blocks=2), 1),
    (dict(window_blocks=65), 2),
    (dict(global_blocks=[0, 0]), 1),
    (dict(global_blocks=[16]), 1),
    (dict(random_blocks=-1), 1),
    (dict(random_blocks=65), 1),
    (dict(num_heads=0), 1),
])
def test_make_layout_rejects(kw, code):
    args = dict(num_heads=2, seq_len=1024, block=64, window_blocks=3, global_blocks=[0], random_blocks=1, seed=0)
    args.update(kw)
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_make_layout(**args)
    assert e.value.status == code
    assert bs.bsattn_last_error()


def test_band_layout_rejects():
    with pytest.raises(bs.BsattnError):
        bs.bsattn_make_band_layout(2, 1024, 64, 1024)
    with pytest.raises(bs.BsattnError):
        bs.bsattn_make_band_layout(2, 1024, 64, -1)


def test_workspace_size_and_destroy():
    lay = bs.bsattn_make_layout(12, 8192, 64, 3, [0, 127], 3, 2)
    n = bs.bsattn_workspace_size(lay, 2, 64)
    # 2 dense rows per head, 128 blocks each -> 8 chunks of 16; slots of 64 x (64+1) floats
    assert n == 2 * 12 * 2 * 8 * 64 * 65 * 4
    assert bs.bsattn_workspace_size(lay, 2, 64, num_routed=64) > n
    with pytest.raises(bs.BsattnError):
        bs.bsattn_workspace_size(lay, 2, 96)
    lay.destroy()
    lay.destroy()                         # idempotent
    bs.lib().bsattn_layout_destroy(None)  # NULL-safe


def test_forward_rejects_before_any_hip_call():
    L = bs.lib()
    lay = bs.bsattn_make_layout(2, 1024, 64, 3, [0], 1, 0)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    ws = ctypes.c_size_t(0)
    # NULL layout
    st = L.bsattn_forward(None, 1, 1, 2, 1024, 64, fake, fake, fake, ctypes.c_void_p(0x2000), fake, None,
                          0.125, None, ws, None)
    assert st == 1
    # H mismatch
    st = L.bsattn_forward(lay.handle, 1, 1, 3, 1024, 64, fake, fake, fake, ctypes.c_void_p(0x2000), fake, None,
                          0.125, None, ws, None)
    assert st == 1 and "match" in bs.bsattn_last_error()
    # unsupported head_dim
    st = L.bsattn_forward(lay.handle, 1, 1, 2, 1024, 96, fake, fake, fake, ctypes.c_void_p(0x2000), fake, None,
                          0.125, None, ws, None)
    assert st == 2
    # misaligned pointer
    st = L.bsattn_forward(lay.handle, 1, 1, 2, 1024, 64, ctypes.c_void_p(0x1002), fake, fake,
                          ctypes.c_void_p(0x2000), fake, None, 0.125, None, ws, None)
    assert st == 1 and "aligned" in bs.bsattn_last_error()
    # out aliasing q
    st = L.bsattn_forward(lay.handle, 1, 1, 2, 1024, 64, fake, fake, fake, fake, fake, None, 0.125, None, ws, None)
    assert st == 1
    # bad scale
    st = L.bsattn_forward(lay.handle, 1, 1, 2, 1024, 64, fake, fake, fake, ctypes.c_void_p(0x2000), fake, None,
                          -1.0, None, ws, None)
    assert st == 1
    # router argument checks
    st = L.bsattn_route_topk(fake, fake, 1, 2, 1024, 64, 0, fake, fake, 1 << 20, None)
    assert st == 1
    st = L.bsattn_route_topk(fake, fake, 1, 2, 16384, 64, 4, fake, fake, 1 << 20, None)
    assert st == 2
    # router workspace: the fp64 scores of every row
    assert bs.bsattn_route_workspace_size(1, 32, 4096, 64) == 32 * 4096 * 8
    assert bs.bsattn_route_workspace_size(2, 3, 1000, 5) == 6 * 1000 * 8
    st = L.bsattn_route_topk(fake, fake, 1, 32, 4096, 128, 64, fake, fake, 32 * 4096 * 8 - 1, None)
    assert st == 1 and "workspace" in bs.bsattn_last_error()
    st = L.bsattn_route_topk(fake, fake, 1, 32, 4096, 128, 64, fake, None, 0, None)
    assert st == 1
    # profile events must be set in pairs
    assert L.bsattn_set_profile_events(fake, None) == 1
    assert L.bsattn_set_profile_events(None, None) == 0


def test_backward_workspace_size_and_lists():
    """Host-side backward work lists: sizes follow the layout's split rows and columns."""
    lay = bs.bsattn_make_layout(12, 8192, 64, 3, [0, 127], 3, 2)
    n = bs.bsattn_backward_workspace_size(lay, 2, 64)
    delta = 2 * 12 * 8192 * 4
    # 2 global rows and 2 global columns per head, each 128 blocks -> 8 chunks of 16
    part = 2 * 12 * 2 * 8 * 64 * 64 * 4
    assert n == delta + part + 2 * part
    assert bs.bsattn_backward_workspace_size(lay, 2, 128) == delta + 3 * 2 * part
    with pytest.raises(bs.BsattnError):
        bs.bsattn_backward_workspace_size(lay, 2, 96)


def test_token_backward_workspace_size():
    """Token layouts: delta, the band and global-row partial slots, then the global
    keys' chunk partials (one chunk per 256 rows at most, about 2048 workgroups)."""
    B, H, L, ng = 2, 3, 4096, 40
    tok = bs.bsattn_make_token_layout(H, L, 64, ng, 4, 7)
    n = bs.bsattn_backward_workspace_size(tok, B, 64)
    delta = B * H * L * 4
    chunks = max(1, min(L // 256, -(-2048 // (B * H * -(-ng // 4)))))   # 4 global keys per workgroup at D = 64
    glob = B * H * ng * chunks * 2 * 64 * 4
    assert n >= delta + glob and n % 256 == 0
    # the global rows' dQ partials grow with B, and so does everything else
    assert bs.bsattn_backward_workspace_size(tok, 2 * B, 64) > n
    assert bs.bsattn_backward_workspace_size(tok, B, 128) > n
    # no global tokens: no global partials, no global-row slots
    tok0 = bs.bsattn_make_token_layout(H, L, 64, 0, 4, 7)
    band = bs.bsattn_make_band_layout(H, L, 64, 64)
    assert bs.bsattn_backward_workspace_size(tok0, B, 64) == bs.bsattn_backward_workspace_size(band, B, 64)


def test_backward_rejects_before_any_hip_call():
    L = bs.lib()
    lay = bs.bsattn_make_layout(2, 1024, 64, 3, [0], 1, 0)
    band = bs.bsattn_make_band_layout(2, 1024, 64, 32)
    tok = bs.bsattn_make_token_layout(2, 1024, 32, 8, 2, 1)
    adp = bs.bsattn_make_adaptive_layout(2, 1024, 4)
    f = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(10)]
    ws = ctypes.c_size_t(0)

    def call(layout, dtype=1, D=64, q=f[0], dq=f[6], dk=f[7], dv=f[8], dout=f[5], scale=0.125, kv=None):
        return L.bsattn_backward(layout, dtype, 1, 2, 1024, D, q, f[1], f[2], f[3], f[4], dout, dq, dk, dv,
                                 kv, scale, None, ws, None)

    assert call(None) == 1
    assert call(adp.handle) == 2 and "layout" in bs.bsattn_last_error()
    assert call(tok.handle, kv=f[9]) == 2 and "padding" in bs.bsattn_last_error()
    assert call(band.handle, kv=f[9]) == 2 and "padding" in bs.bsattn_last_error()
    assert call(lay.handle, dtype=0) == 2 and "bf16" in bs.bsattn_last_error()
    assert call(lay.handle, dout=None) == 1
    assert call(lay.handle, dq=f[0]) == 1 and "alias" in bs.bsattn_last_error()
    assert call(lay.handle, dk=f[6]) == 1 and "alias" in bs.bsattn_last_error()
    assert call(lay.handle, dv=ctypes.c_void_p(0x9002)) == 1 and "aligned" in bs.bsattn_last_error()
    assert call(lay.handle, D=96) == 2
    assert call(lay.handle, scale=0.0) == 1


def test_layer_rejects_before_any_hip_call():
    L = bs.lib()
    lay = bs.bsattn_make_layout(2, 1024, 64, 3, [0], 1, 0)
    adp = bs.bsattn_make_adaptive_layout(2, 1024, 4)
    f = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(8)]
    ws = ctypes.c_size_t(0)

    def call(layout, H=2, D=64, x=f[0], out=f[5], b_qkv=f[2]):
        return L.bsattn_layer_forward(layout, 1, H, 1024, D, x, f[1], b_qkv, f[3], f[4], out, None, 0.125,
                                      None, ws, None)

    assert call(None) == 1
    assert call(adp.handle) == 2 and "layout" in bs.bsattn_last_error()
    assert call(lay.handle, out=f[0]) == 1 and "alias" in bs.bsattn_last_error()
    assert call(lay.handle, b_qkv=ctypes.c_void_p(0x3008)) == 1 and "aligned" in bs.bsattn_last_error()
    assert call(lay.handle, H=3) == 1
    assert call(lay.handle, D=96) == 2
    assert call(lay.handle) == 1 and "workspace" in bs.bsattn_last_error()
    n = bs.bsattn_layer_workspace_size(lay, 1, 64)
    assert n >= 1024 * 128 * (3 * 4 + 4 * 2)


def test_prepare_rejects_before_any_hip_call():
    L = bs.lib()
    lay = bs.bsattn_make_layout(2, 1024, 64, 3, [0], 1, 0)
    adp = bs.bsattn_make_adaptive_layout(2, 1024, 4)
    assert L.bsattn_prepare(None, 1, 64, 0, 0, None) == 1           # NULL layout
    assert L.bsattn_prepare(lay.handle, 0, 64, 0, 0, None) == 1     # batch < 1
    assert L.bsattn_prepare(lay.handle, 1, 96, 0, 0, None) == 2     # head_dim
    assert L.bsattn_prepare(lay.handle, 1, 64, 5, 0, None) == 1     # routed rows need a band layout
    assert L.bsattn_prepare(lay.handle, 1, 64, 2000, 0, None) == 1  # num_routed > seq_len
    assert L.bsattn_prepare(adp.handle, 1, 64, 0, 1, None) == 2     # no backward for adaptive layouts
    assert "backward" in bs.bsattn_last_error()


def test_noalloc_rejects_before_any_hip_call():
    L = bs.lib()
    lay = bs.bsattn_make_layout(2, 1024, 64, 3, [0], 1, 0)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    assert L.bsattn_forward_noalloc(None, 1, 1, 2, 1024, 64, fake, fake, fake, fake, fake, None,
                                    ctypes.c_float(0.125), None) == 1
    assert L.bsattn_forward_noalloc(lay.handle, 1, 1, 2, 1024, 96, fake, fake, fake, fake, fake, None,
                                    ctypes.c_float(0.125), None) == 2


def test_device_build_rejects_token_and_adaptive_layouts():
    L = bs.lib()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    tok = bs.bsattn_make_token_layout(2, 1024, 16, 8, 2, 0)
    ada = bs.bsattn_make_adaptive_layout(2, 1024, 4)
    top = bs.bsattn_make_topr_layout(2, 1024, 100)
    for lay in (tok, ada, top):
        assert L.bsattn_layout_build_device(lay.handle, fake, fake, fake, None) == 2
        assert "device rule" in bs.bsattn_last_error()
    # a layout of 32-token blocks needs the mask array
    sub = bs.bsattn_make_layout(2, 1024, 32, 3, [0], 1, 0)
    assert L.bsattn_layout_build_device(sub.handle, fake, fake, None, None) == 1
    assert "tile_masks_dev" in bs.bsattn_last_error()


def test_candidate_entries_reject_before_any_hip_call():
    L = bs.lib()
    f = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(8)]

    def pos(x=f[0], w=f[1], b=f[2], B=1, Ln=64, C=32, k=32, out=f[3]):
        return L.bsattn_candidate_positions(x, w, b, B, Ln, C, k, out, None)

    assert pos(x=None) == 1
    assert pos(k=0) == 1 and "num_candidates" in bs.bsattn_last_error()
    assert pos(k=65) == 1
    assert pos(C=0) == 1
    assert pos(w=ctypes.c_void_p(0x2002)) == 1 and "aligned" in bs.bsattn_last_error()

    def fwd(dtype=1, D=64, k=32, keep=9, scale=0.125, q=f[0], out=f[4], kept=None):
        return L.bsattn_candidate_forward(dtype, 1, 2, 64, D, q, f[1], f[2], f[3], k, keep, scale, out, f[5],
                                          kept, None)

    assert fwd(dtype=0) == 2 and "bf16" in bs.bsattn_last_error()
    assert fwd(D=96) == 2
    assert fwd(keep=0) == 1 and "keep" in bs.bsattn_last_error()
    assert fwd(keep=33) == 1
    assert fwd(k=65, keep=9) == 1
    assert fwd(scale=0.0) == 1
    assert fwd(q=None) == 1
    assert fwd(out=f[0]) == 1 and "alias" in bs.bsattn_last_error()
    assert fwd(kept=f[3]) == 1 and "alias" in bs.bsattn_last_error()
    assert fwd(out=ctypes.c_void_p(0x5008)) == 1 and "aligned" in bs.bsattn_last_error()
