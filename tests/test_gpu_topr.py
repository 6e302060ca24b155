"""GPU parity of per-query top-keep attention against the oracle.

The kept keys are an integer result: the device's kept-key words must equal
the oracle's mask bit for bit (every query keeps exactly keep_tokens keys,
ties to the lower index).  The forward is compared element by element with
the fp64 oracle at the bf16 tolerances (O 2e-2, LSE 1e-3).  Cases cover the
three selection widths (L <= 2048, <= 4096, <= 8192), D = 64 and 128,
keep = 1 and keep = L, duplicated keys, and the benchmark shape.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from conftest import record_parity
from oracle import topr as OT
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


def _words(mask: np.ndarray) -> np.ndarray:
    """Pack a boolean [..., L] mask into little-endian 64-bit words [..., L/64]."""
    by = np.packbits(mask, axis=-1, bitorder="little")
    return by.reshape(mask.shape[:-1] + (mask.shape[-1] // 8,)).view("<u8")


def _inputs(B, H, L, D, seed):
    g = torch.Generator().manual_seed(seed)
    return tuple(torch.randn((B, H, L, D), generator=g).to(torch.bfloat16) for _ in range(3))


def _select(q, k, keep):
    B, H, L, D = q.shape
    lay = bs.bsattn_make_topr_layout(H, L, keep)
    bs.bsattn_layout_upload(lay)
    bits = bs.bsattn_topr_select(lay, q.cuda(), k.cuda())
    torch.cuda.synchronize()
    return bits.cpu().numpy().view(np.uint64)


def _check_bits(q, k, keep, tag, heads=None, rows=None):
    _say(tag, tuple(q.shape), "keep", keep)
    got = _select(q, k, keep)
    B, H, L, D = q.shape
    pop = np.unpackbits(got.view(np.uint8), axis=-1).reshape(B, H, L, -1).sum(-1)
    assert np.all(pop == keep), f"{tag}: rows keep {np.unique(pop)} keys, want {keep}"
    if rows is not None:
        q32, k32 = OT._as_f32(q), OT._as_f32(k)
        for b, h, t in rows:
            s = OT.ranking_scores(q32[b, h, t][None], k32[b, h])[0]
            m = np.zeros(L, dtype=bool)
            m[OT.kept_keys(s, keep)] = True
            assert np.array_equal(got[b, h, t], _words(m)), f"{tag}: row {(b, h, t)} differs"
        return
    want = _words(OT.topr_mask(q, k, keep, heads=heads))
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            bad = np.argwhere(got[b, h] != want[b, h])
            assert bad.size == 0, f"{tag}: head {(b, h)}: {len(bad)} words differ, first {bad[0].tolist()}"


@pytest.mark.parametrize("B,H,L,D,keep", [
    (1, 2, 512, 64, 153),      # 16 threads per query
    (2, 1, 1024, 128, 307),
    (1, 1, 3072, 64, 921),     # 32 threads per query
    (1, 1, 4096, 128, 1228),
    (1, 2, 320, 64, 1),
    (1, 1, 448, 128, 448),     # keep = L
])
def test_selection_bits_exact(B, H, L, D, keep):
    q, k, _ = _inputs(B, H, L, D, seed=L + D + keep)
    _check_bits(q, k, keep, f"topr bits B{B} H{H} L{L} D{D} keep{keep}")


def test_selection_bits_longest_sampled():
    """64 threads per query (L = 8192): sampled query rows against the oracle."""
    q, k, _ = _inputs(1, 1, 8192, 64, seed=11)
    g = np.random.default_rng(11)
    rows = [(0, 0, t) for t in sorted({0, 1, 4095, 8191, *g.integers(0, 8192, 12).tolist()})]
    _check_bits(q, k, 2457, "topr bits L8192 sampled", rows=rows)


def test_selection_ties_to_lower_index():
    """Key rows repeated in blocks of 8: every score occurs 8 times, so the cut
    falls inside a group of equal scores on most rows."""
    g = torch.Generator().manual_seed(12)
    q = torch.randn((1, 2, 1024, 64), generator=g).to(torch.bfloat16)
    base = torch.randn((1, 2, 128, 64), generator=g)
    k = base.repeat_interleave(8, dim=2).to(torch.bfloat16)
    _check_bits(q, k, 300, "topr bits repeated keys")


def test_selection_integer_scores():
    """Entries in {-1, 0, 1}: integer scores with many ties and -0 / +0 alike."""
    g = torch.Generator().manual_seed(13)
    q = torch.randint(-1, 2, (1, 1, 1024, 64), generator=g).to(torch.bfloat16)
    k = torch.randint(-1, 2, (1, 1, 1024, 64), generator=g).to(torch.bfloat16)
    _check_bits(q, k, 100, "topr bits integer scores")


def _forward_check(q, k, v, keep, tag, heads=None, rows=None):
    _say(tag, tuple(q.shape), "keep", keep)
    B, H, L, D = q.shape
    scale = D ** -0.5
    lay = bs.bsattn_make_topr_layout(H, L, keep)
    bs.bsattn_layout_upload(lay)
    out, lse = bs.forward(q.cuda(), k.cuda(), v.cuda(), lay, scale=scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        ro, rl = OT.topr_attention_forward(q, k, v, keep, scale, rows=rows)
        go = np.stack([o[b, h, t] for b, h, t in rows])
        gl = np.array([l[b, h, t] for b, h, t in rows])
    else:
        ro, rl = OT.topr_attention_forward(q, k, v, keep, scale, heads=heads)
        sel = (slice(None), list(range(H)) if heads is None else list(heads))
        go, gl, ro, rl = o[sel], l[sel], ro[sel], rl[sel]
    eo = float(np.max(np.abs(go - ro)))
    el = float(np.max(np.abs(gl - rl)))
    print(f"  {tag}: O {eo:.2e} / {TOL_O:g}  LSE {el:.2e} / {TOL_LSE:g}", file=sys.stderr, flush=True)
    record_parity(tag, "O", eo, TOL_O)
    record_parity(tag, "LSE", el, TOL_LSE)
    assert eo <= TOL_O and el <= TOL_LSE, f"{tag}: O {eo:.3e} LSE {el:.3e}"


@pytest.mark.parametrize("B,H,L,D,keep", [
    (1, 2, 512, 64, 153),
    (2, 1, 1024, 128, 307),
    (1, 2, 1024, 64, 1),
    (1, 1, 2048, 128, 2048),   # keep = L: dense attention
    (1, 1, 3072, 64, 921),
])
def test_forward_full(B, H, L, D, keep):
    q, k, v = _inputs(B, H, L, D, seed=3 * L + D + keep)
    _forward_check(q, k, v, keep, f"topr fwd B{B} H{H} L{L} D{D} keep{keep}")


def test_benchmark_shape():
    """The benchmark call (B1 H12 L2048 D64, keep 614): kept keys of three whole
    heads, whole-head forward parity on two heads and sampled rows on the rest."""
    wl = WORKLOADS["topr-L2048"]
    inp = make_inputs(wl)
    q, k, v = inp["q"], inp["k"], inp["v"]
    _check_bits(q, k, wl.keep_tokens, "topr-L2048 bits", heads=[0, 5, wl.heads - 1])
    _forward_check(q, k, v, wl.keep_tokens, "topr-L2048 whole heads", heads=[0, wl.heads - 1])
    g = np.random.default_rng(14)
    rows = [(0, h, int(t)) for h in range(1, wl.heads - 1) for t in g.integers(0, wl.seq_len, 4)]
    _forward_check(q, k, v, wl.keep_tokens, "topr-L2048 sampled rows", rows=rows)
