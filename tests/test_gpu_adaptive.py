"""GPU parity of the content-adaptive block layout: the kept key blocks equal
the oracle's bit for bit (an integer decision both sides take from the same
fp64 operations in the same order), and the forward over them equals the
oracle's dense masked attention within the bf16 tolerances (O 2e-2, LSE
1e-3 max-abs).  Small shapes everywhere, the benchmark shape on the whole
selection and on sampled rows."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from oracle import adaptive as OD
from oracle import attention as OA
from conftest import record_parity
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bs.lib()
    yield
    torch.cuda.synchronize()


def _layout(wl):
    lay = bs.bsattn_make_adaptive_layout(wl.heads, wl.seq_len, wl.keep_blocks)
    bs.bsattn_layout_upload(lay)
    return lay


def _check_selection(wl, inp, lay):
    dev = {k: v.cuda() for k, v in inp.items()}
    cols = bs.bsattn_adaptive_select(lay, dev["q"], dev["k"]).cpu().numpy()
    rows = OD.adaptive_rows(inp["q"], inp["k"], wl.keep_blocks)
    want = np.asarray(rows, dtype=np.int32)
    assert cols.shape == want.shape
    assert np.array_equal(cols, want)
    return rows


def _compare(o, l, ro, rl, tag):
    eo = float(np.abs(o - ro).max())
    el = float(np.abs(l - rl).max())
    _say(tag, f"max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    record_parity(tag, "O", eo, TOL_O)
    record_parity(tag, "LSE", el, TOL_LSE)
    assert eo <= TOL_O and el <= TOL_LSE, (tag, eo, el)


def _full(wl, tag):
    _say(tag, wl)
    inp = make_inputs(wl)
    lay = _layout(wl)
    rows = _check_selection(wl, inp, lay)
    dev = {k: v.cuda() for k, v in inp.items()}
    out, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    torch.cuda.synchronize()
    ro, rl, _ = OD.adaptive_attention_forward(inp["q"], inp["k"], inp["v"], wl.keep_blocks, wl.scale, rows=rows)
    _compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, tag)


@pytest.mark.parametrize("D", [64, 128])
def test_adaptive_full(D):
    # 16 blocks a side, 4 kept: rows shorter than a chunk
    _full(WORKLOADS["adaptive-L8192"].with_(batch=2, heads=2, seq_len=1024, head_dim=D, keep_blocks=4),
          f"adaptive L1024 keep 4 D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_adaptive_split_rows(D):
    # 32 blocks a side, 20 kept: every row is split into chunks and merged
    _full(WORKLOADS["adaptive-L8192"].with_(batch=1, heads=2, seq_len=2048, head_dim=D, keep_blocks=20),
          f"adaptive L2048 keep 20 D={D}")


def test_adaptive_edges():
    base = WORKLOADS["adaptive-L8192"].with_(batch=2, heads=1, seq_len=512)
    _full(base.with_(keep_blocks=1), "adaptive keep 1")
    _full(base.with_(keep_blocks=8), "adaptive keep all (dense)")
    _full(base.with_(seq_len=64, keep_blocks=1), "adaptive one block")


def test_adaptive_ties_go_to_the_lower_block():
    # identical key blocks give equal scores: the lowest indices must win
    wl = WORKLOADS["adaptive-L8192"].with_(batch=1, heads=1, seq_len=512, keep_blocks=3)
    inp = make_inputs(wl)
    inp["k"][:] = inp["k"][:, :, :64].repeat(1, 1, 8, 1)
    lay = _layout(wl)
    rows = _check_selection(wl, inp, lay)
    assert all(r == [0, 1, 2] for r in rows[0][0])


def test_adaptive_benchmark_shape():
    wl = WORKLOADS["adaptive-L8192"]
    _say("adaptive bench shape", wl)
    inp = make_inputs(wl)
    lay = _layout(wl)
    rows = _check_selection(wl, inp, lay)
    dev = {k: v.cuda() for k, v in inp.items()}
    out, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    g = np.random.default_rng(8)
    pts = [(int(g.integers(wl.batch)), int(g.integers(wl.heads)), int(t)) for t in g.integers(0, wl.seq_len, 24)]
    pts += [(0, 0, 0), (1, wl.heads - 1, wl.seq_len - 1)]
    for b, h, t in pts:
        mask = np.zeros((1, wl.seq_len), dtype=bool)
        for j in rows[b][h][t // 64]:
            mask[0, 64 * j:64 * j + 64] = True
        ro, rl = OA.masked_attention(inp["q"][b, h, t][None].double().numpy(), inp["k"][b, h].double().numpy(),
                                     inp["v"][b, h].double().numpy(), mask, wl.scale)
        _compare(o[b, h, t][None], l[b, h, t][None], ro, rl, f"adaptive bench row {(b, h, t)}")


def test_adaptive_rejects():
    wl = WORKLOADS["adaptive-L8192"].with_(batch=1, heads=1, seq_len=256, keep_blocks=2)
    lay = _layout(wl)
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"], inp["k"], inp["v"], lay, scale=wl.scale,
                   key_valid_len=torch.tensor([100], dtype=torch.int32, device="cuda"))
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"].float(), inp["k"].float(), inp["v"].float(), lay, scale=wl.scale)
    o, l = bs.forward(inp["q"], inp["k"], inp["v"], lay, scale=wl.scale)
    with pytest.raises(bs.BsattnError):
        bs.backward(inp["q"], inp["k"], inp["v"], o, l, o, lay, scale=wl.scale)
