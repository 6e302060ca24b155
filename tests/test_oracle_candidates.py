"""Pins for the candidate-list oracle (CPU only).

Checked against things other than the oracle itself: torch's Conv1d in fp64
(which taps meet which rows, the padding, the bias), a one-hot weight whose
output is a single input element, a case where the fixed addition order
decides the value, numpy-free rounding cases, a brute-force statement of the
rank rule, and dense masked attention over the candidate set when every
candidate is kept.
"""
import numpy as np
import pytest
import torch

from oracle import candidates as OC


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _case(B=2, L=40, C=24, k=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, L, C), generator=g).to(torch.bfloat16)
    w = torch.randn((k, C, 3), generator=g) * 3.0
    bias = torch.rand((k,), generator=g) * L
    return x, w, bias


def test_conv_matches_torch_conv1d():
    x, w, bias = _case()
    y = OC.conv_outputs(x, w.numpy(), bias.numpy())
    ref = torch.nn.functional.conv1d(x.double().transpose(1, 2), w.double(), bias.double(), padding=1)
    ref = ref.transpose(1, 2).numpy()
    assert y.shape == ref.shape
    assert np.max(np.abs(y - ref)) < 1e-9          # only the addition order differs
    # the first and last tokens see one padded tap each
    assert np.max(np.abs(y[:, 0] - ref[:, 0])) < 1e-9 and np.max(np.abs(y[:, -1] - ref[:, -1])) < 1e-9


def test_one_hot_weight_picks_one_element():
    x, _, _ = _case(B=1, L=12, C=6, k=3, seed=1)
    w = np.zeros((3, 6, 3), dtype=np.float32)
    w[0, 4, 0] = 1.0        # channel 0: x[t - 1, 4]
    w[1, 2, 2] = 1.0        # channel 1: x[t + 1, 2]
    w[2, 5, 1] = 1.0        # channel 2: x[t, 5]
    bias = np.array([0.5, -1.0, 0.0], dtype=np.float32)
    y = OC.conv_outputs(x, w, bias)
    xf = x.double().numpy()[0]
    assert y[0, 0, 0] == 0.5                               # t = 0: the tap before is padding
    assert np.array_equal(y[0, 1:, 0], 0.5 + xf[:-1, 4])
    assert np.array_equal(y[0, :-1, 1], -1.0 + xf[1:, 2])
    assert y[0, -1, 1] == -1.0                             # last token: the tap after is padding
    assert np.array_equal(y[0, :, 2], xf[:, 5])


def test_fixed_addition_order():
    """bias 2^53, then +1 (u = 0), then -2^53 (u = 1): 2^53 + 1 rounds back to
    2^53 in fp64 (ties to even), so the sum is 0; in any order that cancels
    the large terms first it would be 1."""
    x = np.zeros((1, 3, 1))
    x[0, 0, 0] = 1.0
    x[0, 1, 0] = 1.0
    w = np.zeros((1, 1, 3))
    w[0, 0, 0] = 1.0          # tap u = 0 at t = 1 reads x[0] = 1
    w[0, 0, 1] = -(2.0 ** 53)  # tap u = 1 at t = 1 reads x[1] = 1
    bias = np.array([2.0 ** 53])
    y = OC.conv_outputs(x, w, bias)
    assert y[0, 1, 0] == 0.0


def test_positions_round_and_clamp():
    L = 10
    y = np.array([-3.2, -0.5, 0.5, 1.5, 2.5, 2.4999, 9.49, 9.5, 1e30, np.inf, -np.inf, np.nan])
    p = OC.positions_from_outputs(y, L)
    assert p.tolist() == [0, 0, 0, 2, 2, 2, 9, 9, 9, 9, 0, 0]
    assert p.dtype == np.int32


def test_kept_candidates_brute_force():
    g = np.random.default_rng(3)
    for trial in range(40):
        L, D = 30, 16
        q = _bf16(g.integers(-2, 3, (D,)))
        kk = _bf16(g.integers(-2, 3, (L, D)))          # integer scores: many ties
        pos = g.integers(0, L, 12)
        keep = int(g.integers(1, 15))
        got = OC.kept_candidates(q.float().numpy(), kk.float().numpy(), pos, keep)
        cand = sorted(set(pos.tolist()))
        s = {c: float((q.double() * kk[c].double()).sum()) for c in cand}
        want = sorted(c for c in cand if sum(1 for o in cand if s[o] > s[c] or (s[o] == s[c] and o < c)) < keep)
        assert got.tolist() == want, trial


def test_duplicates_collapse_and_small_sets_keep_all():
    q = _bf16(np.ones(8))
    kk = _bf16(np.arange(20 * 8).reshape(20, 8) % 7)
    got = OC.kept_candidates(q.float().numpy(), kk.float().numpy(), [5, 5, 5, 2, 2], 9)
    assert got.tolist() == [2, 5]


def test_keep_all_equals_masked_attention_over_candidates():
    g = torch.Generator().manual_seed(5)
    B, H, L, D, k = 1, 2, 48, 16, 6
    q, kk, v = (torch.randn((B, H, L, D), generator=g).to(torch.bfloat16) for _ in range(3))
    pos = torch.randint(0, L, (B, L, k), generator=g).numpy().astype(np.int32)
    scale = D ** -0.5
    o, lse = OC.candidate_attention_forward(q, kk, v, pos, k, scale)
    for h in range(H):
        mask = torch.zeros((L, L), dtype=torch.bool)
        for t in range(L):
            mask[t, torch.as_tensor(pos[0, t], dtype=torch.long)] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[0, h].double(), kk[0, h].double(), v[0, h].double(), attn_mask=mask, scale=scale)
        assert np.max(np.abs(o[0, h] - ref.numpy())) < 1e-12
        s = scale * (q[0, h].double() @ kk[0, h].double().T)
        s = s.masked_fill(~mask, float("-inf"))
        assert np.max(np.abs(lse[0, h] - torch.logsumexp(s, -1).numpy())) < 1e-12


@pytest.mark.parametrize("keep", [1, 3])
def test_kept_keys_outscore_dropped_candidates(keep):
    g = torch.Generator().manual_seed(keep)
    B, H, L, D, k = 1, 1, 32, 16, 8
    q, kk = (torch.randn((B, H, L, D), generator=g).to(torch.bfloat16) for _ in range(2))
    pos = torch.randint(0, L, (B, L, k), generator=g).numpy()
    m = OC.kept_mask(q, kk, pos, keep)[0, 0]
    s = (q[0, 0].double() @ kk[0, 0].double().T).numpy()
    for t in range(L):
        cand = np.unique(pos[0, t])
        kept = np.flatnonzero(m[t])
        assert len(kept) == min(keep, len(cand)) and set(kept) <= set(cand.tolist())
        dropped = [c for c in cand if c not in set(kept.tolist())]
        if dropped:
            assert s[t, kept].min() >= s[t, dropped].max() - 1e-5
