"""Pins for the oracle's attention gradients (CPU only).

The analytic gradients of ``oracle.attention_grad`` are checked against
things other than themselves: central finite differences of the oracle's
forward (itself pinned to torch's scaled_dot_product_attention), torch
autograd of the dense masked formula in fp64, and invariants that follow from
the softmax: every non-empty row's probabilities sum to one, so the key-sum of
dV is the sum of dO over non-empty rows and the key-sum of dK vanishes;
keys that no row sees and rows that see no key get zero gradient; with one
allowed key per row the softmax is constant, so dQ = dK = 0.  A copy of the
gradient with the softmax Jacobian's row term dropped is shown to fail the
dK invariant, so that pin can catch that mistake.
"""
import numpy as np
import torch

from oracle import attention as OA
from oracle import attention_grad as OG
from oracle import layout as OL


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _small_case(seed):
    n, m, D = 6, 9, 4
    q, k, v, do = _rand((n, D), seed), _rand((m, D), seed + 1), _rand((m, D), seed + 2), _rand((n, D), seed + 3)
    g = np.random.default_rng(seed + 4)
    mask = g.random((n, m)) < 0.5
    mask[np.arange(n - 1), g.integers(0, m, n - 1)] = True
    mask[n - 1] = False                                   # one row with no allowed key
    return q, k, v, do, mask


def test_grad_matches_central_differences():
    q, k, v, do, mask = _small_case(11)
    scale = 0.7
    dq, dk, dv = OG.masked_attention_grad(q, k, v, mask, scale, do)

    def loss(qq, kk, vv):
        o, _ = OA.masked_attention(qq, kk, vv, mask, scale)
        return float((o * do).sum())

    h = 1e-5
    for x, g_an, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        g_num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            g_num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(g_num - g_an).max() < 1e-8, which


def _torch_dense_grad(q, k, v, do, mask, scale):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tm = torch.from_numpy(mask)
    s = scale * (tq @ tk.transpose(-1, -2))
    s = s.masked_fill(~tm, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)                     # rows with no key
    o = p @ tv
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_layout_backward_matches_torch_autograd():
    B, H, L, D = 2, 2, 4 * 64, 16
    q, k, v, do = (_rand((B, H, L, D), s) for s in (21, 22, 23, 24))
    lay = OL.make_layout(H, L, 64, 3, [0], 1, 7)
    valid = [L, 150]
    dq, dk, dv = OG.attention_backward(q, k, v, do, lay, 0.25, valid_len=valid, chunk=100)
    for b in range(B):
        for h in range(H):
            mask = lay.token_mask_rows(h, np.arange(L), valid[b])
            rq, rk, rv = _torch_dense_grad(q[b, h], k[b, h], v[b, h], do[b, h], mask, 0.25)
            assert np.abs(dq[b, h] - rq).max() < 1e-12
            assert np.abs(dk[b, h] - rk).max() < 1e-12
            assert np.abs(dv[b, h] - rv).max() < 1e-12


def _invariants(dq, dk, dv, do, mask):
    nonempty = mask.any(axis=1)
    seen = mask.any(axis=0)
    return (np.abs(dv.sum(axis=0) - do[nonempty].sum(axis=0)).max(),
            np.abs(dk.sum(axis=0)).max(),
            np.abs(dq[~nonempty]).max(initial=0.0),
            max(np.abs(dk[~seen]).max(initial=0.0), np.abs(dv[~seen]).max(initial=0.0)))


def test_softmax_invariants_on_a_padded_layout():
    L, D = 5 * 64, 8
    q, k, v, do = (_rand((L, D), s, 2.0) for s in (31, 32, 33, 34))
    lay = OL.make_layout(1, L, 64, 3, [4], 1, 3)
    mask = lay.token_mask_rows(0, np.arange(L), 200)     # keys 200.. padded
    mask[7] = False                                      # and one row sees nothing
    dq, dk, dv = OG.masked_attention_grad(q, k, v, mask, 0.35, do)
    e_dv, e_dk, e_dq0, e_unseen = _invariants(dq, dk, dv, do, mask)
    assert e_dv < 1e-10 and e_dk < 1e-10
    assert e_dq0 == 0.0 and e_unseen == 0.0


def test_dropped_jacobian_row_term_breaks_the_dk_invariant():
    """Plant the mistake in a copy of the oracle's arithmetic: dS = P * dP."""
    L, D = 3 * 64, 8
    q, k, v, do = (_rand((L, D), s) for s in (41, 42, 43, 44))
    mask = OL.make_layout(1, L, 64, 3, [], 0, 0).token_mask_rows(0, np.arange(L), None)
    scale = 0.3
    p = OG.masked_softmax(scale * (q @ k.T), mask)
    ds_wrong = p * (do @ v.T)
    dk_wrong = scale * (ds_wrong.T @ q)
    assert np.abs(dk_wrong.sum(axis=0)).max() > 1e-3
    _, dk, _ = OG.masked_attention_grad(q, k, v, mask, scale, do)
    assert np.abs(dk.sum(axis=0)).max() < 1e-10


def test_one_key_per_row_has_constant_softmax():
    n, m, D = 10, 12, 5
    q, k, v, do = _rand((n, D), 51), _rand((m, D), 52), _rand((m, D), 53), _rand((n, D), 54)
    cols = np.random.default_rng(55).integers(0, m, n)
    mask = np.zeros((n, m), dtype=bool)
    mask[np.arange(n), cols] = True
    dq, dk, dv = OG.masked_attention_grad(q, k, v, mask, 0.4, do)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    ref = np.zeros((m, D))
    for t in range(n):
        ref[cols[t]] += do[t]
    assert np.abs(dv - ref).max() < 1e-14


def test_band_backward_matches_autograd_and_closed_form():
    """Token band |t - s| <= w (SQA page, section 2.1): the oracle backward over a
    band layout equals torch autograd of the dense formula with the band written
    out directly, and for w = 0 (each query sees only its own key: P = 1) it has
    the closed form dQ = dK = 0, dV = dO."""
    L, D = 3 * 64, 8
    q, k, v, do = (_rand((1, 1, L, D), s) for s in (41, 42, 43, 44))
    t = np.arange(L)
    for w in (0, 5, 70):
        lay = OL.make_band_layout(1, L, 64, w)
        dq, dk, dv = OG.attention_backward(q, k, v, do, lay, 0.3, chunk=50)
        mask = np.abs(t[:, None] - t[None, :]) <= w
        rq, rk, rv = _torch_dense_grad(q[0, 0], k[0, 0], v[0, 0], do[0, 0], mask, 0.3)
        assert np.abs(dq[0, 0] - rq).max() < 1e-12, w
        assert np.abs(dk[0, 0] - rk).max() < 1e-12, w
        assert np.abs(dv[0, 0] - rv).max() < 1e-12, w
        if w == 0:
            assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
            assert np.array_equal(dv, do)


def test_routed_backward_matches_torch_autograd():
    """The routed gradients against torch autograd of the dense formula, with the
    mask written out here by loops: row t sees key s iff t is routed or |t - s| <= band."""
    B, H, L, D = 1, 2, 3 * 64, 8
    band = 20
    q, k, v, do = (_rand((B, H, L, D), s) for s in (31, 32, 33, 34))
    routed = np.array([[[3, 64, 100, 191]], [[0, 5, 6, 150]]]).reshape(B, H, 4)
    dq, dk, dv = OG.routed_attention_backward(q, k, v, do, routed, band, 0.3, chunk=70)
    for h in range(H):
        mask = np.zeros((L, L), dtype=bool)
        for t in range(L):
            for s_ in range(L):
                mask[t, s_] = t in set(routed[0, h].tolist()) or abs(t - s_) <= band
        rq, rk, rv = _torch_dense_grad(q[0, h], k[0, h], v[0, h], do[0, h], mask, 0.3)
        assert np.abs(dq[0, h] - rq).max() < 1e-12
        assert np.abs(dk[0, h] - rk).max() < 1e-12
        assert np.abs(dv[0, h] - rv).max() < 1e-12



def test_token_pattern_backward_matches_torch_autograd():
    """The token-granular pattern's gradients (attention_backward over a TokenLayout)
    against torch autograd of the dense formula, with the mask composed here from its
    four parts: t global, s global, |t - s| <= w, or s one of t's random tokens (the
    random draws themselves are pinned in the token-layout tests)."""
    from oracle import layout as OL
    B, H, L, D = 1, 2, 160, 8
    w, ng, r = 6, 5, 3
    q, k, v, do = (_rand((B, H, L, D), s) for s in (41, 42, 43, 44))
    lay = OL.make_token_layout(H, L, w, ng, r, 9)
    gset = set(lay.global_tokens)
    assert len(gset) == ng
    dq, dk, dv = OG.attention_backward(q, k, v, do, lay, 0.3, chunk=50)
    for h in range(H):
        mask = np.zeros((L, L), dtype=bool)
        for t in range(L):
            links = set(lay.random_links(h, t))
            assert len(links) == (0 if t in gset else r)
            for s_ in range(L):
                mask[t, s_] = t in gset or s_ in gset or abs(t - s_) <= w or s_ in links
        rq, rk, rv = _torch_dense_grad(q[0, h], k[0, h], v[0, h], do[0, h], mask, 0.3)
        assert np.abs(dq[0, h] - rq).max() < 1e-12
        assert np.abs(dk[0, h] - rk).max() < 1e-12
        assert np.abs(dv[0, h] - rv).max() < 1e-12
