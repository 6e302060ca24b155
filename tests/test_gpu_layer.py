"""GPU parity of the attention layer (bsattn_layer_forward) against the fp64
oracle layer (oracle.layer): qkv projection, head split, block-sparse
attention, head concatenation, output projection.

Tolerance: every output element within TOL_REL of the largest output
magnitude.  The HIP path rounds q, k, v, the attention output and the layer
output to bf16 once each (2^-9 relative each) and accumulates the GEMMs in
fp32; measured errors are a few tenths of a percent.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from oracle import layer as OLY
from oracle import layout as OL
from conftest import record_parity
from workloads import WORKLOADS, make_inputs, make_layer_params

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bs.lib()
    yield
    torch.cuda.synchronize()


def _case(wl, tag):
    _say(tag, wl)
    p = make_layer_params(wl)
    vl = make_inputs(wl).get("valid_len") if wl.padded else None
    if wl.token:
        lay = bs.bsattn_make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                          wl.layout_seed)
        olay = OL.make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                    wl.layout_seed)
    elif wl.band:
        lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
        olay = OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    else:
        lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                    wl.random_blocks, wl.layout_seed)
        olay = OL.make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                              wl.random_blocks, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    d = {k: v.cuda() for k, v in p.items()}
    out = bs.layer_forward(d["x"], d["w_qkv"], d["b_qkv"], d["w_proj"], d["b_proj"], lay, wl.heads,
                           key_valid_len=None if vl is None else vl.cuda(), scale=wl.scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = OLY.layer_forward(p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], olay, wl.heads, wl.scale,
                            valid_len=None if vl is None else vl.tolist())
    assert np.isfinite(got).all()
    scale = np.abs(ref).max()
    e = np.abs(got - ref).max() / scale
    _say(tag, "max|ref| %.4g  max|err|/max|ref| %.3e" % (scale, e))
    record_parity(tag, "out (rel)", e, TOL_REL)
    assert e <= TOL_REL, f"{tag}: relative error {e}"


def test_layer_d64():
    _case(WORKLOADS["bigbird-L2048"].with_(batch=2, heads=4, seq_len=1024, global_blocks=(0, 15)), "layer d64")


def test_layer_d128_padded():
    _case(WORKLOADS["window-pad-L16384"].with_(batch=2, heads=2, seq_len=2048), "layer d128 pad")


def test_layer_benchmark_shape():
    _case(WORKLOADS["bigbird-L8192"], "layer bigbird-L8192")


@pytest.mark.parametrize("D", [64, 128])
def test_layer_band(D):
    # token band |t - s| <= 100 (SQA page, section 2.1) inside the layer
    _case(WORKLOADS["band256-L8192"].with_(batch=2, heads=2, seq_len=1024, head_dim=D, band_tokens=100),
          f"layer band D={D}")


def test_layer_block32():
    # 32-token blocks (SQA page, section 5: block sizes) inside the layer
    _case(WORKLOADS["bigbird32-L8192"].with_(batch=1, heads=2, seq_len=2048, global_blocks=(0, 63)),
          "layer block32 L2048")


def test_layer_token_pattern():
    # token-granular BigBird pattern (BigBird page, 核心实现) inside the layer
    _case(WORKLOADS["bigbird-tok-L8192"].with_(batch=2, heads=2, seq_len=1024, num_global=40, random_tokens=4),
          "layer token pattern")
