"""GPU parity over a seeded random sweep of small configurations: every layout kind
(window/global/random rule on 32-, 64- and 128-token blocks, token band, token-granular
pattern, content-adaptive), both head widths, ragged block counts, and the backward of the
rule layouts and the band -- each compared element by element with the fp64 oracle (bf16 tolerances:
O 2e-2 and LSE 1e-3 max-abs; gradients 2e-2 of the reference's max-abs)."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from oracle import adaptive as OD
from oracle import attention as OA
from oracle import attention_grad as OG
from oracle import layout as OL
from conftest import record_parity
from workloads import WORKLOADS, make_grad_output, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bs.lib()
    yield
    torch.cuda.synchronize()


def _cmp(o, l, ro, rl, tag):
    ninf = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l), ninf), tag
    eo = float(np.abs(o - ro).max())
    el = float(np.abs(l[~ninf] - rl[~ninf]).max()) if (~ninf).any() else 0.0
    _say(tag, f"dO={eo:.2e} dLSE={el:.2e}")
    record_parity(tag, "O", eo, 2e-2)
    record_parity(tag, "LSE", el, 1e-3)
    assert eo <= 2e-2 and el <= 1e-3, (tag, eo, el)


def _forward(wl, lay, inp):
    dev = {k: v.cuda() for k, v in inp.items()}
    out, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", range(12))
def test_sweep_rule_layouts(case):
    g = np.random.default_rng(1000 + case)
    block = int(g.choice([32, 64, 128]))
    D = int(g.choice([64, 128]))
    nt = int(g.integers(1, 14))                       # 64-token tiles a side
    L = 64 * nt
    if L % block:
        L = block * (L // block + 1)
    nb = L // block
    w = int(g.integers(0, 4)) * 2 + 1
    ng = int(g.integers(0, min(nb, 3) + 1))
    G = sorted(g.choice(nb, size=ng, replace=False).tolist())
    r = int(g.integers(0, 4))
    wl = WORKLOADS["bigbird-L2048"].with_(batch=int(g.integers(1, 3)), heads=int(g.integers(1, 3)), seq_len=L,
                                          head_dim=D, block=block, window_blocks=w, global_blocks=tuple(G),
                                          random_blocks=r, layout_seed=int(g.integers(0, 2**31)),
                                          data_seed=int(g.integers(0, 2**31)))
    tag = f"rule block={block} D={D} L={L} w={w} G={G} r={r} B={wl.batch} H={wl.heads}"
    _say(tag)
    inp = make_inputs(wl)
    lay = bs.bsattn_make_layout(wl.heads, L, block, w, G, r, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    olay = OL.make_layout(wl.heads, L, block, w, G, r, wl.layout_seed)
    o, l = _forward(wl, lay, inp)
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale)
    _cmp(o, l, ro, rl, tag)
    _backward_check(wl, lay, olay, inp, tag)


def _backward_check(wl, lay, olay, inp, tag):
    """Backward of the same case against the oracle's gradients; each tensor
    within 2e-2 of its largest magnitude (floored at 1e-3: a band of width 0
    has exactly zero dQ and dK)."""
    do = make_grad_output(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    out, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    grads = bs.backward(dev["q"], dev["k"], dev["v"], out, lse, do.cuda(), lay, scale=wl.scale)
    torch.cuda.synchronize()
    refs = OG.attention_backward(inp["q"], inp["k"], inp["v"], do, olay, wl.scale)
    for name, gr, rf in zip(("dQ", "dK", "dV"), grads, refs):
        e = float(np.abs(gr.float().cpu().numpy() - rf).max() / max(np.abs(rf).max(), 1e-3))
        _say(tag, name, f"{e:.2e}")
        record_parity(tag, name + " (rel)", e, 2e-2)
        assert e <= 2e-2, (tag, name, e)


@pytest.mark.parametrize("case", range(6))
def test_sweep_band_and_token(case):
    g = np.random.default_rng(2000 + case)
    D = int(g.choice([64, 128]))
    L = 64 * int(g.integers(1, 12))
    w = int(g.integers(0, min(L, 300)))
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=int(g.integers(1, 3)), heads=int(g.integers(1, 3)), seq_len=L,
                                              head_dim=D, band_tokens=w, data_seed=int(g.integers(0, 2**31)))
    inp = make_inputs(wl)
    # band layout
    tag = f"band D={D} L={L} w={w}"
    _say(tag)
    lay = bs.bsattn_make_band_layout(wl.heads, L, 64, w)
    bs.bsattn_layout_upload(lay)
    o, l = _forward(wl, lay, inp)
    olay = OL.make_band_layout(wl.heads, L, 64, w)
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale)
    _cmp(o, l, ro, rl, tag)
    _backward_check(wl, lay, olay, inp, tag + " bwd")
    # token pattern
    ng = int(g.integers(0, min(L, 100) + 1))
    r = int(g.integers(0, 10))
    seed = int(g.integers(0, 2**31))
    tag = f"token D={D} L={L} w={w} ng={ng} r={r}"
    _say(tag)
    lay = bs.bsattn_make_token_layout(wl.heads, L, w, ng, r, seed)
    bs.bsattn_layout_upload(lay)
    o, l = _forward(wl, lay, inp)
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], OL.make_token_layout(wl.heads, L, w, ng, r, seed),
                                  wl.scale)
    _cmp(o, l, ro, rl, tag)


@pytest.mark.parametrize("case", range(6))
def test_sweep_adaptive(case):
    g = np.random.default_rng(3000 + case)
    D = int(g.choice([64, 128]))
    nb = int(g.integers(1, 40))
    keep = int(g.integers(1, nb + 1))
    wl = WORKLOADS["adaptive-L8192"].with_(batch=int(g.integers(1, 3)), heads=int(g.integers(1, 3)), seq_len=64 * nb,
                                           head_dim=D, keep_blocks=keep, data_seed=int(g.integers(0, 2**31)))
    tag = f"adaptive D={D} nb={nb} keep={keep}"
    _say(tag)
    inp = make_inputs(wl)
    lay = bs.bsattn_make_adaptive_layout(wl.heads, wl.seq_len, keep)
    bs.bsattn_layout_upload(lay)
    dev = {k: v.cuda() for k, v in inp.items()}
    cols = bs.bsattn_adaptive_select(lay, dev["q"], dev["k"]).cpu().numpy()
    rows = OD.adaptive_rows(inp["q"], inp["k"], keep)
    assert np.array_equal(cols, np.asarray(rows, dtype=np.int32)), tag
    o, l = _forward(wl, lay, inp)
    ro, rl, _ = OD.adaptive_attention_forward(inp["q"], inp["k"], inp["v"], keep, wl.scale, rows=rows)
    _cmp(o, l, ro, rl, tag)
