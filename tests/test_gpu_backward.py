"""GPU parity of the backward pass: the HIP path through the C ABI against the
fp64 oracle gradients (oracle.attention_grad).

Inputs Q, K, V and dO are seeded bf16 draws (workloads.make_inputs,
make_grad_output).  The HIP backward runs on the HIP forward's O and LSE, as a
training step would; one case instead feeds the oracle's own O (rounded to
bf16) and LSE (rounded to fp32) to test the backward alone.

Tolerance: every element of dQ, dK and dV within TOL_REL of the largest
magnitude of that reference tensor (bf16 rounding of P, dS, O and the outputs
each contribute about 2^-9 relative; see the backward tolerance derivation in
the design notes).  Small shapes are compared everywhere; the benchmark shape
(B=2, H=12, L=8192) is compared on one whole (batch, head) pair.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from oracle import attention as OA
from oracle import attention_grad as OG
from oracle import layout as OL
from conftest import record_parity
from workloads import WORKLOADS, make_grad_output, make_inputs

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


def _layouts(wl):
    lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                wl.random_blocks, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    olay = OL.make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                          wl.random_blocks, wl.layout_seed)
    return lay, olay


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _compare(got, ref, what):
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        scale = max(np.abs(r).max(), 1e-6)
        e = np.abs(g - r).max() / scale
        errs.append(e)
        _say(what, name, "max|ref| %.4g  max|err|/max|ref| %.3e" % (scale, e))
        record_parity(what, name + " (rel)", e, TOL_REL)
        assert e <= TOL_REL, f"{what}: {name} relative error {e}"
    return errs


def _hip_backward(wl, inp, do, lay, o=None, lse=None):
    dev = {k: v.cuda() for k, v in inp.items()}
    vl = dev.get("valid_len")
    if o is None:
        o, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, key_valid_len=vl, scale=wl.scale)
    dq, dk, dv = bs.backward(dev["q"], dev["k"], dev["v"], o, lse, do.cuda(), lay, key_valid_len=vl,
                             scale=wl.scale)
    torch.cuda.synchronize()
    return _f64(dq), _f64(dk), _f64(dv)


def _band_layouts(wl):
    lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    bs.bsattn_layout_upload(lay)
    return lay, OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)


def _case(wl, tag, heads=None, batches=None, layouts=_layouts):
    _say(tag, wl)
    inp = make_inputs(wl)
    do = make_grad_output(wl)
    lay, olay = layouts(wl)
    got = _hip_backward(wl, inp, do, lay)
    vl = inp.get("valid_len")
    ref = OG.attention_backward(inp["q"], inp["k"], inp["v"], do, olay, wl.scale,
                                valid_len=None if vl is None else vl.tolist(), heads=heads, batches=batches)
    if heads is not None or batches is not None:
        bsel = list(range(wl.batch)) if batches is None else list(batches)
        hsel = list(range(wl.heads)) if heads is None else list(heads)
        got = tuple(x[np.ix_(bsel, hsel)] for x in got)
        ref = tuple(x[np.ix_(bsel, hsel)] for x in ref)
    return _compare(got, ref, tag)


def test_backward_d64_split_rows_and_columns():
    # 32 blocks a side: the global rows and columns (32 blocks) are split in two chunks
    wl = WORKLOADS["bigbird-L2048"].with_(batch=2, heads=2)
    _case(wl, "bwd d64 L2048")


def test_backward_d128():
    wl = WORKLOADS["bigbird-L2048"].with_(batch=1, heads=2, head_dim=128, data_seed=7)
    _case(wl, "bwd d128 L2048")


def test_backward_key_padding_d128():
    wl = WORKLOADS["window-pad-L16384"].with_(batch=2, heads=2, seq_len=2048)
    _case(wl, "bwd pad d128 L2048")


def test_backward_key_padding_d64():
    wl = WORKLOADS["bigbird-L2048"].with_(batch=3, heads=1, padded=True, data_seed=11)
    _case(wl, "bwd pad d64 L2048")


def test_backward_alone_on_oracle_forward():
    """The backward fed the oracle's O (bf16) and LSE (fp32) instead of the HIP forward's."""
    wl = WORKLOADS["bigbird-L2048"].with_(batch=1, heads=2, data_seed=5)
    _say("bwd alone", wl)
    inp = make_inputs(wl)
    do = make_grad_output(wl)
    lay, olay = _layouts(wl)
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale)
    o = torch.from_numpy(ro).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(rl).to(torch.float32).cuda()
    got = _hip_backward(wl, inp, do, lay, o=o, lse=lse)
    ref = OG.attention_backward(inp["q"], inp["k"], inp["v"], do, olay, wl.scale)
    _compare(got, ref, "bwd alone")


def test_backward_workspace_dirty_and_reused():
    wl = WORKLOADS["bigbird-L2048"].with_(batch=1, heads=2, data_seed=9)
    _say("bwd dirty workspace", wl)
    inp = make_inputs(wl)
    do = make_grad_output(wl).cuda()
    lay, olay = _layouts(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    o, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    n = bs.bsattn_backward_workspace_size(lay, wl.batch, wl.head_dim)
    ws = torch.full(((n + 255) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        dq, dk, dv = bs.backward(dev["q"], dev["k"], dev["v"], o, lse, do, lay, scale=wl.scale, workspace=ws)
        torch.cuda.synchronize()
        outs.append((_f64(dq), _f64(dk), _f64(dv)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    ref = OG.attention_backward(inp["q"], inp["k"], inp["v"], do.cpu(), olay, wl.scale)
    _compare(outs[0], ref, "bwd dirty workspace")


def test_backward_benchmark_shape_one_head():
    wl = WORKLOADS["bigbird-L8192"]
    _case(wl, "bwd bigbird-L8192 (b=1, h=5)", heads=[5], batches=[1])


def test_backward_rows_with_no_key():
    """Window-only layout with heavy padding: rows past the window of the valid
    keys see no key (LSE = -inf) and must get zero dQ; keys past the valid
    length get zero dK and dV."""
    wl = WORKLOADS["bigbird-L2048"].with_(batch=2, heads=2, seq_len=1024, global_blocks=(), random_blocks=0,
                                          padded=True, data_seed=13)
    _say("bwd empty rows", wl)
    inp = make_inputs(wl)
    inp["valid_len"] = torch.tensor([100, 1024], dtype=torch.int32)
    do = make_grad_output(wl)
    lay, olay = _layouts(wl)
    got = _hip_backward(wl, inp, do, lay)
    ref = OG.attention_backward(inp["q"], inp["k"], inp["v"], do, olay, wl.scale, valid_len=[100, 1024])
    assert (got[0][0, :, 3 * 64:] == 0).all()          # rows of blocks >= 3 see no valid key
    assert (got[1][0, :, 100:] == 0).all() and (got[2][0, :, 100:] == 0).all()
    _compare(got, ref, "bwd empty rows")


def test_backward_block128():
    _case(WORKLOADS["bigbird128-L8192"].with_(batch=1, heads=2, seq_len=2048, global_blocks=(0, 15)),
          "bwd block128 L2048")


def test_backward_block128_padded():
    _case(WORKLOADS["bigbird128-L8192"].with_(batch=2, heads=2, seq_len=2048, global_blocks=(0, 15), padded=True),
          "bwd block128 L2048 padded")


@pytest.mark.parametrize("D", [64, 128])
def test_backward_block32(D):
    _case(WORKLOADS["bigbird32-L8192"].with_(batch=1, heads=2, seq_len=2048, head_dim=D, global_blocks=(0, 63)),
          f"bwd block32 L2048 D={D}")


# Token band |t - s| <= band (SQA page, section 2.1): narrow bands, bands that
# cut through tiles, and a band wide enough that rows and columns are split.
@pytest.mark.parametrize("band,D,L", [(37, 64, 1536), (128, 64, 1536), (256, 64, 1536), (600, 64, 2048),
                                      (64, 128, 1536), (200, 128, 1536)])
def test_backward_band(band, D, L):
    wl = WORKLOADS["band256-L8192"].with_(batch=2, heads=2, seq_len=L, head_dim=D, band_tokens=band)
    _case(wl, f"bwd band {band} D={D} L={L}", layouts=_band_layouts)


def test_backward_band_benchmark_shape_one_head():
    wl = WORKLOADS["band256-L8192"]
    _case(wl, "bwd band256-L8192 (b=0, h=3)", heads=[3], batches=[0], layouts=_band_layouts)


def test_backward_band_rejects_padding():
    wl = WORKLOADS["band256-L8192"].with_(batch=1, heads=1, seq_len=512, band_tokens=64)
    lay, _ = _band_layouts(wl)
    dev = {k: v.cuda() for k, v in make_inputs(wl).items()}
    o, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    vl = torch.tensor([300], dtype=torch.int32, device="cuda")
    with pytest.raises(bs.BsattnError, match="padding"):
        bs.backward(dev["q"], dev["k"], dev["v"], o, lse, torch.ones_like(o), lay, key_valid_len=vl, scale=wl.scale)


# ---------------- routed-query variant ----------------

def _routed_bwd_case(wl, tag, heads=None):
    """bsattn_backward_routed against the oracle's routed gradients: the routed rows
    come from the device router (bit-exact with the oracle's), the forward's O and
    LSE from bsattn_forward_routed."""
    from oracle import router as OR
    _say(tag, wl)
    inp = make_inputs(wl)
    do = make_grad_output(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    k = wl.routed_k
    rr = torch.empty((wl.batch, wl.heads, k), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(dev["q"], dev["w"], k, rr)
    band = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    bs.bsattn_layout_upload(band)
    o, lse = bs.forward_routed(dev["q"], dev["k"], dev["v"], band, rr, scale=wl.scale)
    dq, dk, dv = bs.backward_routed(dev["q"], dev["k"], dev["v"], o, lse, do.cuda(), band, rr, scale=wl.scale)
    torch.cuda.synchronize()
    want_rows = OR.topk_rows(OR.router_scores(inp["q"], inp["w"]), k)
    assert np.array_equal(rr.cpu().numpy(), want_rows), f"{tag}: routed rows differ"
    got = (_f64(dq), _f64(dk), _f64(dv))
    ref = OG.routed_attention_backward(inp["q"], inp["k"], inp["v"], do, want_rows, wl.band_tokens, wl.scale,
                                       heads=heads)
    if heads is not None:
        got = tuple(x[:, list(heads)] for x in got)
        ref = tuple(x[:, list(heads)] for x in ref)
    return _compare(got, ref, tag)


def test_backward_routed_small_d128():
    wl = WORKLOADS["routed-L4096"].with_(heads=2, seq_len=512)
    _routed_bwd_case(wl, "bwd routed L512 D128 k64 band32")


def test_backward_routed_d64_ragged_k():
    # 70 routed rows: two routed tiles, the second with 6 rows
    wl = WORKLOADS["routed-L4096"].with_(batch=2, heads=2, seq_len=1024, head_dim=64, routed_k=70, band_tokens=100)
    _routed_bwd_case(wl, "bwd routed L1024 D64 k70 band100")


def test_backward_routed_wide_band_split_rows():
    # band 512 at L = 2048: band rows of up to 17 blocks are split (dQ partials
    # summed before the routed rows are rewritten) and so are the columns
    wl = WORKLOADS["routed-L4096"].with_(heads=2, seq_len=2048, head_dim=64, band_tokens=512)
    _routed_bwd_case(wl, "bwd routed L2048 D64 k64 band512")


def test_backward_routed_full_size_heads():
    """The routed workload's own shape (B1 H32 L4096 D128, band 32, top 64): whole heads."""
    wl = WORKLOADS["routed-L4096"]
    _routed_bwd_case(wl, "bwd routed-L4096 heads 0, 13, 31", heads=[0, 13, 31])


# ---------------- token-granular BigBird pattern ----------------
# Query t sees key s iff t or s is global, |t - s| <= w, or s is one of t's
# random tokens (BigBird page, code example).  The band and the global rows go
# through the block passes; each non-global row's global keys outside its
# band and its random tokens through the token kernels.

def _token_layouts(wl):
    lay = bs.bsattn_make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                      wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    olay = OL.make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                wl.layout_seed)
    return lay, olay


@pytest.mark.parametrize("D", [64, 128])
def test_backward_token_pattern(D):
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=2, heads=2, seq_len=1536, head_dim=D)
    _case(wl, f"bwd token L1536 D={D}", layouts=_token_layouts)


@pytest.mark.parametrize("D,w,ng,r", [(64, 5, 77, 8), (128, 200, 77, 3), (64, 130, 150, 16)])
def test_backward_token_many_globals(D, w, ng, r):
    # 5-10% global tokens: two or three global-row tiles, global keys inside and outside the band
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=1, heads=2, seq_len=1536, head_dim=D, band_tokens=w,
                                              num_global=ng, random_tokens=r, layout_seed=D + w)
    _case(wl, f"bwd token w={w} ng={ng} r={r} D={D}", layouts=_token_layouts)


def test_backward_token_wide_band_split():
    # a 600-token band at L = 2048: band rows and columns of up to 21 blocks are split
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=1, heads=2, seq_len=2048, band_tokens=600, num_global=20)
    _case(wl, "bwd token w=600 L2048", layouts=_token_layouts)


def test_backward_token_edges():
    base = WORKLOADS["bigbird-tok-L8192"].with_(batch=2, heads=2, seq_len=256, head_dim=64)
    _case(base.with_(num_global=0), "bwd token: no global tokens", layouts=_token_layouts)
    _case(base.with_(random_tokens=0), "bwd token: no random tokens", layouts=_token_layouts)
    _case(base.with_(num_global=1, band_tokens=0), "bwd token: one global token, window 0", layouts=_token_layouts)
    _case(base.with_(seq_len=128, num_global=128), "bwd token: every token global", layouts=_token_layouts)
    _case(base.with_(seq_len=64, num_global=2, band_tokens=63, random_tokens=64), "bwd token: one tile",
          layouts=_token_layouts)


def test_backward_token_benchmark_shape_one_head():
    wl = WORKLOADS["bigbird-tok-L8192"]
    _case(wl, "bwd bigbird-tok-L8192 (b=1, h=5)", heads=[5], batches=[1], layouts=_token_layouts)


def test_backward_token_rejects_padding():
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=1, heads=1, seq_len=256)
    lay, _ = _token_layouts(wl)
    dev = {k: v.cuda() for k, v in make_inputs(wl).items()}
    o, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    vl = torch.tensor([100], dtype=torch.int32, device="cuda")
    with pytest.raises(bs.BsattnError, match="padding"):
        bs.backward(dev["q"], dev["k"], dev["v"], o, lse, torch.ones_like(o), lay, key_valid_len=vl, scale=wl.scale)
