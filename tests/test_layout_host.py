"""The library's host layout builder equals the oracle's layout bit for bit
(integer work: exact equality), on every workload and on random parameter
tuples.  Host code only -- no GPU call."""
import numpy as np
import pytest

import block_sparse_transformer_amd as bs
from oracle import layout as OL
from workloads import WORKLOADS


def _both(H, L, w, G, r, seed):
    lay = bs.bsattn_make_layout(H, L, 64, w, list(G), r, seed)
    got = bs.bsattn_layout_csr(lay)
    want = OL.make_layout(H, L, 64, w, list(G), r, seed).csr()
    return got, want


@pytest.mark.parametrize("name", [n for n, wl in WORKLOADS.items()
                                  if not (wl.routed or wl.band or wl.token or wl.adaptive or wl.topr or wl.candidates)
                                  and wl.block == 64])
def test_workload_layouts_bit_exact(name):
    wl = WORKLOADS[name]
    (rp, ci), (orp, oci) = _both(wl.heads, wl.seq_len, wl.window_blocks, wl.global_blocks,
                                 wl.random_blocks, wl.layout_seed)
    assert rp.dtype == np.int32 and ci.dtype == np.int32
    assert np.array_equal(rp, orp)
    assert np.array_equal(ci, oci)


def test_band_layout_bit_exact():
    wl = WORKLOADS["routed-L4096"]
    lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    rp, ci = bs.bsattn_layout_csr(lay)
    orp, oci = OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens).csr()
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    wl = WORKLOADS["band256-L8192"]
    lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    rp, ci = bs.bsattn_layout_csr(lay)
    orp, oci = OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens).csr()
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    for band in (0, 1, 63, 64, 65, 200):
        lay = bs.bsattn_make_band_layout(2, 16 * 64, 64, band)
        rp, ci = bs.bsattn_layout_csr(lay)
        orp, oci = OL.make_band_layout(2, 16 * 64, 64, band).csr()
        assert np.array_equal(rp, orp) and np.array_equal(ci, oci), band


def test_random_parameter_tuples_bit_exact():
    g = np.random.default_rng(1234)
    for _ in range(300):
        nb = int(g.integers(1, 40))
        H = int(g.integers(1, 4))
        w = int(g.integers(0, 8)) * 2 + 1
        ng = int(g.integers(0, min(nb, 5) + 1))
        G = sorted(g.choice(nb, size=ng, replace=False).tolist())
        r = int(g.integers(0, 12))
        seed = int(g.integers(0, 2 ** 63)) * (1 if g.random() < 0.5 else 2) % (2 ** 64)
        (rp, ci), (orp, oci) = _both(H, nb * 64, w, G, r, seed)
        assert np.array_equal(rp, orp), (nb, H, w, G, r, seed)
        assert np.array_equal(ci, oci), (nb, H, w, G, r, seed)


def test_global_order_does_not_matter():
    a = bs.bsattn_layout_csr(bs.bsattn_make_layout(2, 2048, 64, 3, [31, 0, 7], 2, 5))
    b = bs.bsattn_layout_csr(bs.bsattn_make_layout(2, 2048, 64, 3, [0, 7, 31], 2, 5))
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_large_seed_and_head_values():
    (rp, ci), (orp, oci) = _both(3, 64 * 64, 5, [0, 63], 7, (1 << 64) - 1)
    assert np.array_equal(ci, oci)


def _expand(rows_ptr, cols, f):
    """A block-f*64 CSR expanded to 64-token tiles (each block -> f x f tiles)."""
    out_ptr, out_col = [0], []
    for r in range(len(rows_ptr) - 1):
        row = cols[rows_ptr[r]:rows_ptr[r + 1]]
        for _ in range(f):
            out_col.extend(f * int(j) + b for j in row for b in range(f))
            out_ptr.append(len(out_col))
    return np.asarray(out_ptr, dtype=np.int32), np.asarray(out_col, dtype=np.int32)


def test_block128_layouts_are_the_rule_on_128_blocks_expanded_to_tiles():
    g = np.random.default_rng(99)
    for _ in range(60):
        nb = int(g.integers(1, 24))
        H = int(g.integers(1, 3))
        w = int(g.integers(0, 5)) * 2 + 1
        ng = int(g.integers(0, min(nb, 3) + 1))
        G = sorted(g.choice(nb, size=ng, replace=False).tolist())
        r = int(g.integers(0, 6))
        seed = int(g.integers(0, 2**63))
        lay = bs.bsattn_make_layout(H, nb * 128, 128, w, G, r, seed)
        rp, ci = bs.bsattn_layout_csr(lay)
        orp, oci = OL.make_layout(H, nb * 128, 128, w, G, r, seed).csr()
        erp, eci = _expand(orp, oci, 2)
        assert np.array_equal(rp, erp) and np.array_equal(ci, eci), (nb, H, w, G, r, seed)


def _quarters(rp, ci, masks, H, nt):
    """[H, 2nt, 2nt] bool: the 32-token block mask the tiles and quarter masks describe."""
    m = np.zeros((H, 2 * nt, 2 * nt), dtype=bool)
    for r in range(H * nt):
        h, i = divmod(r, nt)
        for e in range(rp[r], rp[r + 1]):
            j, q = int(ci[e]), int(masks[e])
            assert 0 < q < 16
            for a in range(2):
                for b in range(2):
                    m[h, 2 * i + a, 2 * j + b] = bool((q >> (2 * a + b)) & 1)
    return m


def test_block32_layouts_are_the_rule_on_32_blocks_as_tile_quarters():
    g = np.random.default_rng(32)
    for _ in range(60):
        nt = int(g.integers(1, 12))
        nb = 2 * nt
        H = int(g.integers(1, 3))
        w = int(g.integers(0, 5)) * 2 + 1
        ng = int(g.integers(0, min(nb, 3) + 1))
        G = sorted(g.choice(nb, size=ng, replace=False).tolist())
        r = int(g.integers(0, 6))
        seed = int(g.integers(0, 2**63))
        lay = bs.bsattn_make_layout(H, nt * 64, 32, w, G, r, seed)
        rp, ci = bs.bsattn_layout_csr(lay)
        masks = bs.bsattn_layout_tile_masks(lay)
        assert masks is not None and masks.dtype == np.uint8 and masks.shape == ci.shape
        assert rp.shape == (H * nt + 1,)
        for row in range(H * nt):   # tiles ascending and unique within a row
            assert np.all(np.diff(ci[rp[row]:rp[row + 1]]) > 0)
        olay = OL.make_layout(H, nt * 64, 32, w, G, r, seed)
        want = np.stack([olay.block_mask(h) for h in range(H)])
        assert np.array_equal(_quarters(rp, ci, masks, H, nt), want), (nt, H, w, G, r, seed)


def test_tile_masks_absent_for_64_and_128_blocks():
    assert bs.bsattn_layout_tile_masks(bs.bsattn_make_layout(2, 512, 64, 3, [0], 1, 7)) is None
    assert bs.bsattn_layout_tile_masks(bs.bsattn_make_layout(2, 512, 128, 3, [0], 1, 7)) is None


def test_block32_rejects_lengths_that_are_not_whole_tiles():
    with pytest.raises(RuntimeError):
        bs.bsattn_make_layout(1, 32 * 5, 32, 3, [], 0, 1)


def _token_rows_match(H, L, w, ng, r, seed, rows=None):
    lay = bs.bsattn_make_token_layout(H, L, w, ng, r, seed)
    g, links = bs.bsattn_layout_token_links(lay)
    olay = OL.make_token_layout(H, L, w, ng, r, seed)
    assert g.tolist() == olay.global_tokens
    assert links.shape == (H, L, r)
    for h, t in (rows if rows is not None else [(h, t) for h in range(H) for t in range(L)]):
        want = olay.random_links(h, t)
        got = [int(x) for x in links[h, t] if x >= 0]
        assert got == want, (H, L, w, ng, r, seed, h, t)
        assert np.all(links[h, t, len(got):] == -1)
    return lay


def test_token_layout_random_tokens_bit_exact():
    g = np.random.default_rng(17)
    for _ in range(12):
        L = 64 * int(g.integers(1, 9))
        w = int(g.integers(0, min(L, 150)))
        ng = int(g.integers(0, min(L, 40) + 1))
        r = int(g.integers(0, 12))
        _token_rows_match(int(g.integers(1, 3)), L, w, ng, r, int(g.integers(0, 2**63)))


def test_token_layout_edge_cases():
    _token_rows_match(1, 64, 63, 64, 8, 1)        # every token global: no random tokens at all
    _token_rows_match(1, 128, 60, 1, 64, 2)       # fewer candidates than r near the middle rows
    _token_rows_match(2, 256, 0, 0, 5, 3)         # no window beyond the diagonal, no global tokens


def test_token_layout_benchmark_shape_sampled_rows():
    from workloads import WORKLOADS
    wl = WORKLOADS["bigbird-tok-L8192"]
    g = np.random.default_rng(4)
    rows = [(int(g.integers(wl.heads)), int(t)) for t in g.integers(0, wl.seq_len, 40)]
    rows += [(0, 0), (0, wl.seq_len - 1), (wl.heads - 1, 1170), (3, 1171)]
    _token_rows_match(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens, wl.layout_seed,
                      rows=rows)


def test_token_layout_csr_is_band_tiles_then_gathered_tiles():
    lay = bs.bsattn_make_token_layout(2, 640, 70, 70, 3, 9)
    rp, ci = bs.bsattn_layout_csr(lay)
    nb, n_gt = 10, 2
    for r in range(2 * nb):
        i = r % nb
        lo, hi = max(0, 64 * i - 70) // 64, min(639, 64 * i + 63 + 70) // 64
        assert ci[rp[r]:rp[r + 1]].tolist() == list(range(lo, hi + 1)) + [nb + c for c in range(n_gt)]


def test_token_layout_rejects():
    for args in [(1, 100, 3, 2, 2, 0), (1, 256, 256, 2, 2, 0), (1, 256, 3, 257, 2, 0), (1, 256, 3, 2, 65, 0),
                 (0, 256, 3, 2, 2, 0), (1, 8192, 3, 2049, 2, 0)]:
        with pytest.raises(RuntimeError):
            bs.bsattn_make_token_layout(*args)


def test_adaptive_layout_skeleton():
    lay = bs.bsattn_make_adaptive_layout(3, 640, 4)
    rp, ci = bs.bsattn_layout_csr(lay)
    assert rp.tolist() == [4 * r for r in range(31)]
    assert ci.tolist() == [0, 1, 2, 3] * 30
    assert bs.bsattn_workspace_size(lay, 2, 64) > 2 * 3 * 10 * 64 * 8 * 2


def test_adaptive_layout_rejects():
    for args in [(1, 640, 0), (1, 640, 11), (1, 100, 1), (0, 640, 1), (1, 64 * 1025, 1)]:
        with pytest.raises(RuntimeError):
            bs.bsattn_make_adaptive_layout(*args)
