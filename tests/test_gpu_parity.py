"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (max-abs over every compared element): fp32 inputs 1e-4 on O and
LSE; bf16 inputs 2e-2 on O and 1e-3 on LSE.  Positions of -inf in LSE must
match exactly; block layouts and routed rows are integers and must match
bit for bit.  Small shapes are compared everywhere; the full workload sizes,
in the launch configuration the benchmark times, are compared on sampled
rows evaluated one by one by the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from oracle import attention as OA
from oracle import layout as OL
from oracle import router as OR
from conftest import record_parity
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-3)}


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


def _run(wl, inp, lay):
    dev = {k: v.cuda() for k, v in inp.items()}
    vl = dev.get("valid_len")
    out, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, key_valid_len=vl, scale=wl.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare(o, l, ro, rl, dtype, what=""):
    to, tl = TOL[dtype]
    ninf_g, ninf_r = np.isneginf(l), np.isneginf(rl)
    assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf LSE positions differ"
    fin = ~ninf_r
    eo = np.abs(o - ro).max() if o.size else 0.0
    el = np.abs(l[fin] - rl[fin]).max() if fin.any() else 0.0
    _say(what, f"max|dO|={eo:.3e} (tol {to}) max|dLSE|={el:.3e} (tol {tl})")
    record_parity(what, "O", eo, to)
    record_parity(what, "LSE", el, tl)
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    assert eo <= to, f"{what}: max |dO| = {eo}"
    assert el <= tl, f"{what}: max |dLSE| = {el}"
    return eo, el


def _full_check(wl, tag):
    _say(tag, wl)
    inp = make_inputs(wl)
    lay, olay = _layouts(wl)
    o, l = _run(wl, inp, lay)
    vl = inp.get("valid_len")
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale,
                                  valid_len=None if vl is None else vl.tolist())
    return _compare(o, l, ro, rl, wl.dtype, tag)


def _sample_rows(wl, valid_len=None, n_random=48, seed=0):
    g = np.random.default_rng(seed)
    L, nb = wl.seq_len, wl.num_blocks
    rows = []
    for b in range(wl.batch):
        for h in sorted({0, wl.heads - 1, int(g.integers(0, wl.heads))}):
            ts = {0, 63, 64, L - 1, L - 64, 65}
            for gb in wl.global_blocks:
                ts |= {gb * wl.block, gb * wl.block + 37 % wl.block, gb * wl.block + wl.block - 1}
            if valid_len is not None:
                v = int(valid_len[b])
                ts |= {max(0, v - 1), min(L - 1, v), max(0, v - 65)}
            ts |= set(int(x) for x in g.integers(0, L, n_random // 4))
            rows += [(b, h, t) for t in sorted(ts)]
    return rows


def _sampled_check(wl, tag, seed=0):
    _say(tag, wl)
    inp = make_inputs(wl)
    lay, olay = _layouts(wl)
    o, l = _run(wl, inp, lay)
    vl = inp.get("valid_len")
    rows = _sample_rows(wl, None if vl is None else vl.tolist(), seed=seed)
    ro, rl = OA.attention_rows(inp["q"], inp["k"], inp["v"], olay, wl.scale, rows,
                               valid_len=None if vl is None else vl.tolist())
    go = np.stack([o[b, h, t] for b, h, t in rows])
    gl = np.array([l[b, h, t] for b, h, t in rows])
    return _compare(go, gl, ro, rl, wl.dtype, tag)


# ---------------- the five workloads ----------------

def test_tiny_f32_full():
    _full_check(WORKLOADS["tiny-f32-L512"], "tiny-f32-L512 full")


def test_tiny_recipe_in_bf16_full():
    _full_check(WORKLOADS["tiny-f32-L512"].with_(dtype="bf16", batch=2), "tiny recipe bf16")


def test_bigbird_L2048_reduced_full():
    _full_check(WORKLOADS["bigbird-L2048"].with_(batch=2, heads=3), "bigbird-L2048 B2 H3 full")


def test_bigbird_L2048_full_size_sampled():
    _sampled_check(WORKLOADS["bigbird-L2048"], "bigbird-L2048 full size, sampled rows")


def test_bigbird_L8192_full_size_sampled():
    _sampled_check(WORKLOADS["bigbird-L8192"], "bigbird-L8192 full size, sampled rows")


def _pairs_check(wl, pairs, tag):
    """Every element of the given (b, h) pairs, from one call on the whole workload."""
    _say(tag, wl, pairs)
    inp = make_inputs(wl)
    lay, olay = _layouts(wl)
    o, l = _run(wl, inp, lay)
    vl = inp.get("valid_len")
    for b, h in pairs:
        ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale,
                                      valid_len=None if vl is None else vl.tolist(), heads=[h], batches=[b])
        _compare(o[b, h], l[b, h], ro[b, h], rl[b, h], wl.dtype, f"{tag} (b={b}, h={h})")


def test_bigbird_L8192_whole():
    # the benchmark's own call: B=2, H=12, L=8192, every element of every (b, h)
    _full_check(WORKLOADS["bigbird-L8192"], "bigbird-L8192 whole, B2 H12 (the benchmark call)")


def test_bigbird_L2048_whole():
    _full_check(WORKLOADS["bigbird-L2048"], "bigbird-L2048 whole, B8 H12")


def test_window_pad_L16384_whole_pairs():
    # three whole (b, h) pairs of the full-size call: the shortest and the
    # longest valid length, and one between
    wl = WORKLOADS["window-pad-L16384"]
    vl = make_inputs(wl)["valid_len"].tolist()
    order = sorted(range(wl.batch), key=lambda b: vl[b])
    pairs = [(order[0], 0), (order[-1], wl.heads - 1), (order[len(order) // 2], wl.heads // 2)]
    _pairs_check(wl, pairs, "window-pad-L16384 whole pairs")


def test_bigbird_L8192_one_head_full():
    _full_check(WORKLOADS["bigbird-L8192"].with_(batch=1, heads=1), "bigbird-L8192 B1 H1 full")


def test_window_pad_reduced_full():
    wl = WORKLOADS["window-pad-L16384"].with_(batch=3, heads=2, seq_len=2048)
    _full_check(wl, "window-pad L2048 B3 H2 full")


def test_window_pad_full_size_sampled():
    _sampled_check(WORKLOADS["window-pad-L16384"], "window-pad-L16384 full size, sampled rows")


# ---------------- routed-query variant ----------------

def _routed_case(wl, tag, full=True, seed=0):
    _say(tag, wl)
    inp = make_inputs(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    k = wl.routed_k
    rr = torch.empty((wl.batch, wl.heads, k), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(dev["q"], dev["w"], k, rr)
    torch.cuda.synchronize()
    want = OR.topk_rows(OR.router_scores(inp["q"], inp["w"]), k)
    got = rr.cpu().numpy()
    assert np.array_equal(got, want), f"{tag}: routed rows differ"
    band = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    bs.bsattn_layout_upload(band)
    out, lse = bs.forward_routed(dev["q"], dev["k"], dev["v"], band, rr, scale=wl.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if full:
        ro, rl = OA.routed_attention_forward(inp["q"], inp["k"], inp["v"], want, wl.band_tokens, wl.scale)
        return _compare(o, l, ro, rl, wl.dtype, tag)
    g = np.random.default_rng(seed)
    rows = []
    for b in range(wl.batch):
        for h in sorted({0, wl.heads - 1, int(g.integers(0, wl.heads))}):
            ts = set(want[b, h, :8].tolist()) | {int(want[b, h, -1])}
            ts |= {0, 1, 31, 32, 33, 63, 64, wl.seq_len - 1, wl.seq_len - 33}
            ts |= set(int(x) for x in g.integers(0, wl.seq_len, 12))
            rows += [(b, h, t) for t in sorted(ts)]
    ro, rl = OA.routed_attention_forward(inp["q"], inp["k"], inp["v"], want, wl.band_tokens, wl.scale,
                                         rows=rows)
    go = np.stack([o[b, h, t] for b, h, t in rows])
    gl = np.array([l[b, h, t] for b, h, t in rows])
    return _compare(go, gl, ro, rl, wl.dtype, tag)


def test_routed_full_size_sampled():
    _routed_case(WORKLOADS["routed-L4096"], "routed-L4096 full size, sampled rows", full=False)


def test_routed_reduced_full():
    _routed_case(WORKLOADS["routed-L4096"].with_(heads=3, seq_len=1024), "routed L1024 H3 full")


def test_routed_ragged_k():
    for k in (1, 70, 130):
        _routed_case(WORKLOADS["routed-L4096"].with_(heads=2, seq_len=1024, routed_k=k, batch=2),
                     f"routed ragged k={k}")


def test_routed_L4096_whole():
    _routed_case(WORKLOADS["routed-L4096"], "routed-L4096 whole, B1 H32", full=True)


def test_routed_wide_band_split_rows():
    # a 512-token band splits the band rows into chunks: the band rows' merge and
    # the routed rows' merge both write routed tokens inside those blocks
    for d in (128, 64):
        wl = WORKLOADS["routed-L4096"].with_(heads=2, seq_len=2048, band_tokens=512, head_dim=d, batch=1)
        _routed_case(wl, f"routed band 512 D={d}")


def test_routed_head_dim_64():
    _routed_case(WORKLOADS["routed-L4096"].with_(heads=2, seq_len=1024, head_dim=64, batch=1),
                 "routed D=64")


# ---------------- layout on the device, determinism ----------------

@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.block == 64 and not (w.token or w.adaptive or w.topr or w.candidates)])
def test_device_layout_equals_host(name):
    wl = WORKLOADS[name]
    _say("device layout", name)
    if wl.routed or wl.band:
        lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    else:
        lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                    wl.random_blocks, wl.layout_seed)
    rp, ci = bs.bsattn_layout_csr(lay)
    drp = torch.full((rp.size,), -7, dtype=torch.int32, device="cuda")
    dci = torch.full((max(1, ci.size),), -7, dtype=torch.int32, device="cuda")
    bs.bsattn_layout_build_device(lay, drp, dci)
    torch.cuda.synchronize()
    assert np.array_equal(drp.cpu().numpy(), rp)
    assert np.array_equal(dci.cpu().numpy()[: ci.size], ci)


def test_device_layout_random_tuples():
    g = np.random.default_rng(77)
    for _ in range(40):
        nb = int(g.integers(1, 60))
        H = int(g.integers(1, 4))
        w = int(g.integers(0, 10)) * 2 + 1
        ng = int(g.integers(0, min(nb, 6) + 1))
        G = sorted(g.choice(nb, size=ng, replace=False).tolist())
        r = int(g.integers(0, 20))
        seed = int(g.integers(0, 2 ** 62))
        lay = bs.bsattn_make_layout(H, nb * 64, 64, w, G, r, seed)
        rp, ci = bs.bsattn_layout_csr(lay)
        drp = torch.empty((rp.size,), dtype=torch.int32, device="cuda")
        dci = torch.empty((max(1, ci.size),), dtype=torch.int32, device="cuda")
        bs.bsattn_layout_build_device(lay, drp, dci)
        torch.cuda.synchronize()
        assert np.array_equal(drp.cpu().numpy(), rp), (nb, H, w, G, r, seed)
        assert np.array_equal(dci.cpu().numpy()[: ci.size], ci), (nb, H, w, G, r, seed)


@pytest.mark.parametrize("block", [32, 128])
def test_device_layout_other_block_sizes(block):
    """32- and 128-token blocks: the device rule's tile CSR (and, for 32-token
    blocks, the quarter masks) equal the host's, on the workloads' own layouts
    and random tuples."""
    g = np.random.default_rng(block)
    cases = [WORKLOADS[f"bigbird{block}-L8192"]]
    for _ in range(30):
        nbr = int(g.integers(2, 80 if block == 32 else 40)) // 2 * 2   # rule blocks, an even count
        nbr = max(nbr, 2)
        H = int(g.integers(1, 4))
        w = int(g.integers(0, 8)) * 2 + 1
        ng = int(g.integers(0, min(nbr, 5) + 1))
        G = sorted(g.choice(nbr, size=ng, replace=False).tolist())
        r = int(g.integers(0, 12))
        cases.append((H, nbr * block, w, G, r, int(g.integers(0, 2 ** 62))))
    for c in cases:
        if isinstance(c, tuple):
            H, L, w, G, r, seed = c
        else:
            H, L, w, G, r, seed = c.heads, c.seq_len, c.window_blocks, list(c.global_blocks), c.random_blocks, \
                c.layout_seed
        _say("device layout", block, H, L, w, G, r)
        lay = bs.bsattn_make_layout(H, L, block, w, G, r, seed)
        rp, ci = bs.bsattn_layout_csr(lay)
        masks = bs.bsattn_layout_tile_masks(lay)
        drp = torch.full((rp.size,), -7, dtype=torch.int32, device="cuda")
        dci = torch.full((max(1, ci.size),), -7, dtype=torch.int32, device="cuda")
        dsub = torch.full((max(1, ci.size),), 0xEE, dtype=torch.uint8, device="cuda") if block == 32 else None
        bs.bsattn_layout_build_device(lay, drp, dci, dsub)
        torch.cuda.synchronize()
        assert np.array_equal(drp.cpu().numpy(), rp), c
        assert np.array_equal(dci.cpu().numpy()[: ci.size], ci), c
        if block == 32:
            assert np.array_equal(dsub.cpu().numpy()[: ci.size], masks), c


def test_bitwise_deterministic():
    wl = WORKLOADS["bigbird-L8192"]
    _say("determinism", wl.name)
    dev = make_inputs(wl, device="cuda")
    lay, _ = _layouts(wl)
    o1, l1 = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    o2, l2 = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


# ---------------- edge cases ----------------

def _edge(H, L, D, dtype, w, G, r, seed, B=1, valid=None, qmul=1.0, tag="", rows=None):
    _say("edge", tag, dict(H=H, L=L, D=D, dtype=dtype, w=w, G=G, r=r, B=B, valid=valid))
    g = torch.Generator().manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = (torch.randn(B, H, L, D, generator=g) * qmul).to(dt)
    k = torch.randn(B, H, L, D, generator=g).to(dt)
    v = torch.randn(B, H, L, D, generator=g).to(dt)
    lay = bs.bsattn_make_layout(H, L, 64, w, G, r, seed)
    bs.bsattn_layout_upload(lay)
    olay = OL.make_layout(H, L, 64, w, G, r, seed)
    vl = None if valid is None else torch.tensor(valid, dtype=torch.int32)
    out, lse = bs.forward(q.cuda(), k.cuda(), v.cuda(), lay, key_valid_len=None if vl is None else vl.cuda(),
                          scale=D ** -0.5)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        ro, rl = OA.attention_rows(q, k, v, olay, D ** -0.5, rows, valid_len=valid)
        go = np.stack([o[b, h, t] for b, h, t in rows])
        gl = np.array([l[b, h, t] for b, h, t in rows])
        return _compare(go, gl, ro, rl, dtype, tag)
    ro, rl = OA.attention_forward(q, k, v, olay, D ** -0.5, valid_len=valid)
    return _compare(o, l, ro, rl, dtype, tag)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_edge_single_and_two_blocks(dtype, D):
    _edge(2, 64, D, dtype, 1, [], 0, 1, tag="nb=1")
    _edge(2, 128, D, dtype, 3, [1], 2, 2, tag="nb=2")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_window_covers_all_and_all_global(dtype):
    _edge(2, 6 * 64, 64, dtype, 15, [], 0, 3, tag="window >= nb")
    _edge(2, 5 * 64, 64, dtype, 1, [0, 1, 2, 3, 4], 0, 4, tag="all global")


def test_edge_random_exceeds_candidates():
    _edge(3, 10 * 64, 64, "bf16", 3, [0], 50, 5, tag="r > candidates")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_edge_ragged_padding_and_empty(dtype, D):
    L = 40 * 64
    _edge(2, L, D, dtype, 5, [0], 2, 6, B=4, valid=[L, 1000, 1, 2047], tag="ragged valid_len")
    _edge(2, 8 * 64, D, dtype, 3, [], 1, 7, B=2, valid=[0, 100], tag="valid_len 0: every row empty")


@pytest.mark.parametrize("D", [64, 128])
def test_edge_peaky_logits_late_max(D):
    # large logits whose row maximum appears in a late tile (global row spanning many chunks)
    _edge(2, 48 * 64, D, "bf16", 3, [0, 47], 3, 8, B=2, qmul=8.0, tag="peaky logits")


def test_edge_long_global_rows_many_chunks():
    # 600 blocks per side: global rows need more than 32 chunks of 16 -> larger chunks
    L = 600 * 64
    rows = [(0, 0, t) for t in (0, 1, 31, 63, L - 64, L - 1, 64, 5000, 20000, 38000)]
    _edge(1, L, 64, "bf16", 3, [0, 599], 1, 9, tag="nb=600 global rows", rows=rows)


def test_workspace_dirty_and_reused():
    """The workspace needs no initialisation: a buffer full of NaN serves, and one buffer
    serves consecutive calls with identical results."""
    wl = WORKLOADS["bigbird-L2048"].with_(batch=2, heads=2)
    _say("workspace reuse", wl)
    inp = make_inputs(wl)
    lay, olay = _layouts(wl)
    dev = {k: v.cuda() for k, v in inp.items()}
    n = bs.bsattn_workspace_size(lay, wl.batch, wl.head_dim)
    ws = torch.full(((n + 255) // 4,), float("nan"), dtype=torch.float32, device="cuda")   # dirty
    outs = []
    for _ in range(3):
        out, lse = bs.forward(dev["q"], dev["k"], dev["v"], lay, scale=wl.scale, workspace=ws)
        outs.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l.view(torch.int32), outs[0][1].view(torch.int32))
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale)
    _compare(outs[-1][0].float().cpu().numpy().astype(np.float64), outs[-1][1].cpu().numpy().astype(np.float64),
             ro, rl, "bf16", "workspace reuse")


# ---------------- token-granular window (band layout through the plain forward) ----------------

def _band_layouts(wl):
    lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    bs.bsattn_layout_upload(lay)
    return lay, OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)


@pytest.mark.parametrize("band,D", [(128, 64), (256, 64), (37, 64), (64, 128), (200, 128)])
def test_band_window_full(band, D):
    wl = WORKLOADS["band256-L8192"].with_(batch=2, heads=2, seq_len=1024 + 512, head_dim=D, band_tokens=band)
    _say("band window", band, D)
    inp = make_inputs(wl)
    lay, olay = _band_layouts(wl)
    o, l = _run(wl, inp, lay)
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale)
    _compare(o, l, ro, rl, wl.dtype, f"band {band} D={D}")


def test_band_window_benchmark_shape_sampled():
    wl = WORKLOADS["band256-L8192"]
    _say("band window bench shape", wl)
    inp = make_inputs(wl)
    lay, olay = _band_layouts(wl)
    o, l = _run(wl, inp, lay)
    g = np.random.default_rng(3)
    rows = [(int(g.integers(wl.batch)), int(g.integers(wl.heads)), int(t))
            for t in list(g.integers(0, wl.seq_len, 60)) + [0, 255, 256, wl.seq_len - 1]]
    ro, rl = OA.attention_rows(inp["q"], inp["k"], inp["v"], olay, wl.scale, rows)
    go = np.stack([o[b, h, t] for b, h, t in rows])
    gl = np.array([l[b, h, t] for b, h, t in rows])
    _compare(go, gl, ro, rl, wl.dtype, "band bench shape")


def test_band_rejects_padding_and_fp32():
    wl = WORKLOADS["band256-L8192"].with_(batch=1, heads=1, seq_len=512)
    lay, _ = _band_layouts(wl)
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"], inp["k"], inp["v"], lay, key_valid_len=torch.tensor([300], dtype=torch.int32,
                   device="cuda"))
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"].float(), inp["k"].float(), inp["v"].float(), lay)


# ---------------- 128-token blocks ----------------

def test_block128_full():
    _full_check(WORKLOADS["bigbird128-L8192"].with_(batch=2, heads=2, seq_len=2048, global_blocks=(0, 15)),
                "block128 L2048 full")


def test_block128_padded():
    _full_check(WORKLOADS["bigbird128-L8192"].with_(batch=2, heads=2, seq_len=2048, global_blocks=(0, 15),
                                                    padded=True), "block128 L2048 padded")


def test_block128_benchmark_shape_sampled():
    _sampled_check(WORKLOADS["bigbird128-L8192"], "bigbird128-L8192 full size, sampled rows")


# ---------------- 32-token blocks (tiles with quarter masks) ----------------

@pytest.mark.parametrize("D", [64, 128])
def test_block32_full(D):
    _full_check(WORKLOADS["bigbird32-L8192"].with_(batch=2, heads=2, seq_len=2048, head_dim=D,
                                                   global_blocks=(0, 63)), f"block32 L2048 D={D} full")


def test_block32_ragged_rule():
    # one 64-token tile a side, window wider than the sequence, and rows whose
    # random blocks leave one query half of a tile with no key half in it
    _full_check(WORKLOADS["bigbird32-L8192"].with_(batch=1, heads=3, seq_len=64, global_blocks=()),
                "block32 L64")
    _full_check(WORKLOADS["bigbird32-L8192"].with_(batch=1, heads=3, seq_len=40 * 64, window_blocks=1,
                                                   global_blocks=(5,), random_blocks=1, layout_seed=11),
                "block32 window 1")


def test_block32_benchmark_shape_sampled():
    _sampled_check(WORKLOADS["bigbird32-L8192"], "bigbird32-L8192 full size, sampled rows")


def test_block32_rejects_padding_and_fp32():
    wl = WORKLOADS["bigbird32-L8192"].with_(batch=1, heads=1, seq_len=512, global_blocks=(0,))
    lay, _ = _layouts(wl)
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    vl = torch.tensor([100], dtype=torch.int32, device="cuda")
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"], inp["k"], inp["v"], lay, key_valid_len=vl, scale=wl.scale)
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"].float(), inp["k"].float(), inp["v"].float(), lay, scale=wl.scale)


# ---------------- token-granular BigBird pattern ----------------

def _token_layouts(wl):
    lay = bs.bsattn_make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                      wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    olay = OL.make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                wl.layout_seed)
    return lay, olay


def _token_full(wl, tag):
    _say(tag, wl)
    inp = make_inputs(wl)
    lay, olay = _token_layouts(wl)
    o, l = _run(wl, inp, lay)
    ro, rl = OA.attention_forward(inp["q"], inp["k"], inp["v"], olay, wl.scale)
    _compare(o, l, ro, rl, wl.dtype, tag)


@pytest.mark.parametrize("D", [64, 128])
def test_token_pattern_full(D):
    _token_full(WORKLOADS["bigbird-tok-L8192"].with_(batch=2, heads=2, seq_len=1536, head_dim=D),
                f"token pattern L1536 D={D}")


@pytest.mark.parametrize("D,w,ng,r", [(64, 5, 77, 8), (128, 200, 77, 3), (64, 130, 150, 16)])
def test_token_pattern_many_globals(D, w, ng, r):
    # 5-10% global tokens: several gathered tiles, globals inside and outside the window
    _token_full(WORKLOADS["bigbird-tok-L8192"].with_(batch=1, heads=2, seq_len=1536, head_dim=D, band_tokens=w,
                                                     num_global=ng, random_tokens=r, layout_seed=D + w),
                f"token pattern w={w} ng={ng} r={r} D={D}")


def test_token_pattern_edges():
    base = WORKLOADS["bigbird-tok-L8192"].with_(batch=2, heads=2, seq_len=256, head_dim=64)
    _token_full(base.with_(num_global=0), "token: no global tokens")
    _token_full(base.with_(random_tokens=0), "token: no random tokens")
    _token_full(base.with_(num_global=1, band_tokens=0), "token: one global token, window 0")
    _token_full(base.with_(seq_len=128, num_global=128), "token: every token global")
    _token_full(base.with_(seq_len=64, num_global=2, band_tokens=63, random_tokens=64), "token: one tile")


def test_token_pattern_benchmark_shape_sampled():
    wl = WORKLOADS["bigbird-tok-L8192"]
    _say("token pattern bench shape", wl)
    inp = make_inputs(wl)
    lay, olay = _token_layouts(wl)
    o, l = _run(wl, inp, lay)
    g = np.random.default_rng(6)
    ts = list(g.integers(0, wl.seq_len, 40)) + [0, 1, 63, 64, 1169, 1170, 1171, 8190, 8191]
    rows = [(int(g.integers(wl.batch)), int(g.integers(wl.heads)), int(t)) for t in ts]
    ro, rl = OA.attention_rows(inp["q"], inp["k"], inp["v"], olay, wl.scale, rows)
    go = np.stack([o[b, h, t] for b, h, t in rows])
    gl = np.array([l[b, h, t] for b, h, t in rows])
    _compare(go, gl, ro, rl, wl.dtype, "token pattern bench shape")


def test_token_pattern_rejects():
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=1, heads=1, seq_len=256)
    lay, _ = _token_layouts(wl)
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"], inp["k"], inp["v"], lay, scale=wl.scale,
                   key_valid_len=torch.tensor([100], dtype=torch.int32, device="cuda"))
    with pytest.raises(bs.BsattnError):
        bs.forward(inp["q"].float(), inp["k"].float(), inp["v"].float(), lay, scale=wl.scale)


def test_global_rows_merged_in_kernel():
    """At 128 blocks a side a global row splits into 8 chunks of 16 tiles; the D = 64
    schedule gives each such row a workgroup whose 8 waves hold its chunks and merge it
    at their end.  Every row of both global blocks is compared, plus rows around them."""
    wl = WORKLOADS["bigbird-L8192"].with_(batch=1, heads=2)
    _say("in-kernel merge of global rows", wl)
    inp = make_inputs(wl)
    lay, olay = _layouts(wl)
    o, l = _run(wl, inp, lay)
    ts = list(range(0, 64)) + list(range(wl.seq_len - 64, wl.seq_len)) + [64, 65, 127, 4000, 8127]
    rows = [(0, h, t) for h in range(wl.heads) for t in ts]
    ro, rl = OA.attention_rows(inp["q"], inp["k"], inp["v"], olay, wl.scale, rows)
    go = np.stack([o[b, h, t] for b, h, t in rows])
    gl = np.array([l[b, h, t] for b, h, t in rows])
    _compare(go, gl, ro, rl, wl.dtype, "global rows merged in kernel")


def test_two_chunk_rows_merged_in_kernel():
    """At 32 blocks a side a global row splits into 2 chunks; with 8 batch entries and 12
    heads every XCD holds 24 such rows, and the D = 64 schedule gives four of them to each
    merging workgroup.  Every row of both global blocks of several (b, h) pairs is compared."""
    wl = WORKLOADS["bigbird-L2048"]
    _say("in-kernel merge of 2-chunk rows", wl)
    inp = make_inputs(wl)
    lay, olay = _layouts(wl)
    o, l = _run(wl, inp, lay)
    ts = list(range(0, 64)) + list(range(wl.seq_len - 64, wl.seq_len)) + [64, 1000]
    rows = [(b, h, t) for b, h in [(0, 0), (3, 5), (7, 11), (5, 8)] for t in ts]
    ro, rl = OA.attention_rows(inp["q"], inp["k"], inp["v"], olay, wl.scale, rows)
    go = np.stack([o[b, h, t] for b, h, t in rows])
    gl = np.array([l[b, h, t] for b, h, t in rows])
    _compare(go, gl, ro, rl, wl.dtype, "2-chunk rows merged in kernel")
