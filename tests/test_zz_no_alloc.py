"""The allocation-free forward (bsattn_forward_noalloc) against bsattn_forward.

Both run the same kernels on the same schedule, so the outputs must agree bit
for bit.  Two calls in a row, the second on a smaller input, so that the
second reads the library's scratch array as the first left it."""
import sys

import pytest
import torch

import block_sparse_transformer_amd as bs
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def _case(wl):
    _say("noalloc", wl.name, wl.batch, wl.heads, wl.seq_len, wl.head_dim)
    inp = make_inputs(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                wl.random_blocks, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    B, H, L, D = dev["q"].shape
    bs.bsattn_prepare(lay, B, D)
    ref_o, ref_l = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((B, H, L), float("nan"), dtype=torch.float32, device="cuda")
    bs.bsattn_forward_noalloc(lay, dev["q"], dev["k"], dev["v"], out, lse, scale=wl.scale)
    torch.cuda.synchronize()
    assert bs.bsattn_workspace_size(lay, B, D) > 0          # the case uses the scratch
    assert torch.equal(out, ref_o), f"{wl.name}: O differs from bsattn_forward"
    assert torch.equal(lse, ref_l), f"{wl.name}: LSE differs from bsattn_forward"
    return lay


def test_noalloc_matches_forward_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # split global rows (32 blocks > 16 per chunk) in both; the second call is smaller
    big = WORKLOADS["bigbird-L2048"].with_(batch=3, heads=4)
    small = WORKLOADS["bigbird-L2048"].with_(batch=1, heads=2, seq_len=1536, global_blocks=(0, 23))
    _case(big)
    _case(small)


def test_noalloc_refuses_an_unprepared_shape():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = WORKLOADS["bigbird-L2048"].with_(batch=1, heads=2)
    inp = make_inputs(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                wl.random_blocks, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_forward_noalloc(lay, dev["q"], dev["k"], dev["v"], out, lse, scale=wl.scale)
    assert e.value.status == 5 and "bsattn_prepare" in str(e.value)
