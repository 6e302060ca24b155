"""Pins for the oracle's attention layer (CPU only).

The split of the width-3C projection into (q, k, v) x heads and the
concatenation of the heads are checked by construction: identity projections
turn the layer into the oracle attention on x itself, and a V projection that
is zero with bias c makes every output row equal c's projection whatever Q and
K are.  A copy of the split with the (3, H) order swapped fails the first pin.
"""
import numpy as np

from oracle import attention as OA
from oracle import layer as OLY
from oracle import layout as OL


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_identity_projections_give_attention_on_x():
    B, L, H, D = 2, 3 * 64, 4, 8
    C = H * D
    x = _rand((B, L, C), 1)
    lay = OL.make_layout(H, L, 64, 3, [0], 1, 5)
    w_qkv = np.concatenate([np.eye(C)] * 3, axis=0)
    out = OLY.layer_forward(x, w_qkv, np.zeros(3 * C), np.eye(C), np.zeros(C), lay, H, 0.3)
    xh = x.reshape(B, L, H, D).transpose(0, 2, 1, 3)
    o, _ = OA.attention_forward(xh, xh, xh, lay, 0.3)
    ref = o.transpose(0, 2, 1, 3).reshape(B, L, C)
    assert np.abs(out - ref).max() < 1e-12


def test_constant_values_pass_straight_to_the_output_projection():
    B, L, H, D = 1, 2 * 64, 2, 16
    C = H * D
    x = _rand((B, L, C), 2)
    w_qkv = _rand((3 * C, C), 3)
    w_qkv[2 * C:] = 0.0                                   # V projection weight 0
    b_qkv = _rand(3 * C, 4)
    w_proj, b_proj = _rand((C, C), 5), _rand(C, 6)
    lay = OL.make_layout(H, L, 64, 1, [], 0, 0)
    out = OLY.layer_forward(x, w_qkv, b_qkv, w_proj, b_proj, lay, H, 0.25)
    ref = b_qkv[2 * C:] @ w_proj.T + b_proj               # every row attends at least itself
    assert np.abs(out - ref[None, None, :]).max() < 1e-12


def test_swapped_split_order_is_caught():
    B, L, H, D = 1, 64, 4, 4
    C = H * D
    x = _rand((B, L, C), 7)
    lay = OL.make_layout(H, L, 64, 1, [], 0, 0)
    w_qkv = _rand((3 * C, C), 8)
    good = OLY.layer_forward(x, w_qkv, np.zeros(3 * C), np.eye(C), np.zeros(C), lay, H, 0.5)
    # read the width-3C row as (H, 3, D) instead of (3, H, D)
    qkv = (x @ w_qkv.T).reshape(B, L, H, 3, D)
    q, k, v = (np.ascontiguousarray(qkv[:, :, :, s].transpose(0, 2, 1, 3)) for s in range(3))
    o, _ = OA.attention_forward(q, k, v, lay, 0.5)
    wrong = o.transpose(0, 2, 1, 3).reshape(B, L, C)
    assert np.abs(good - wrong).max() > 1e-3
