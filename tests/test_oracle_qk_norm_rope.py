"""Pins of the QK-RMSNorm + rotary-embedding oracle (CPU only).

Checked against things other than the oracle itself: torch's RMSNorm routine, closed
forms (the mean square after an affine-free norm, rotations by a quarter turn, norms kept
by every rotation), the defining property of rotary embeddings (the dot product of two
rotated vectors depends only on the difference of their positions), the complex-number
form of the interleaved convention, and the channel permutation that maps one pair
convention onto the other.
"""

import math

import numpy as np
import pytest
import torch

from chunk_windowed_softmax_amd.workloads import make_rope_tables
from oracle import qk_norm_rope_reference, rms_norm, rope


def _x(L, H, d, seed=0, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(L, H, d, generator=g, dtype=torch.float64) * scale).numpy()


@pytest.mark.parametrize("affine", [False, True])
def test_rms_norm_matches_torch(affine):
    x = _x(5, 3, 64, seed=1, scale=3.0)
    w = np.linspace(0.5, 1.5, 64) if affine else None
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), None if w is None else torch.from_numpy(w),
                                        eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(x, w, 1e-6), want, rtol=1e-13, atol=1e-14)


def test_affine_free_mean_square_closed_form():
    # mean(y^2) = ms / (ms + eps) for y = x / sqrt(ms + eps)
    x = _x(4, 2, 128, seed=2, scale=0.01)
    eps = 1e-4
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(rms_norm(x, None, eps) ** 2, axis=-1), ms / (ms + eps), rtol=1e-12)


@pytest.mark.parametrize("interleaved", [False, True])
def test_quarter_turn(interleaved):
    y = _x(3, 2, 8, seed=3)
    cos = np.zeros((3, 4))
    sin = np.ones((3, 4))
    out = rope(y, cos, sin, interleaved)
    if interleaved:
        np.testing.assert_array_equal(out[..., 0::2], -y[..., 1::2])
        np.testing.assert_array_equal(out[..., 1::2], y[..., 0::2])
    else:
        np.testing.assert_array_equal(out[..., :4], -y[..., 4:])
        np.testing.assert_array_equal(out[..., 4:], y[..., :4])


def test_zero_angle_is_identity():
    y = _x(3, 2, 16, seed=4)
    np.testing.assert_array_equal(rope(y, np.ones((3, 8)), np.zeros((3, 8))), y)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_keeps_pair_norms(interleaved):
    L, d = 6, 64
    y = _x(L, 3, d, seed=5)
    cos, sin = make_rope_tables(L, d)
    out = rope(y, cos.numpy(), sin.numpy(), interleaved)
    if interleaved:
        n_in = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
        n_out = out[..., 0::2] ** 2 + out[..., 1::2] ** 2
    else:
        n_in = y[..., :d // 2] ** 2 + y[..., d // 2:] ** 2
        n_out = out[..., :d // 2] ** 2 + out[..., d // 2:] ** 2
    # the fp32 tables are unit vectors up to fp32 rounding
    np.testing.assert_allclose(n_out, n_in, rtol=1e-6)


@pytest.mark.parametrize("interleaved", [False, True])
def test_dot_product_depends_on_position_difference(interleaved):
    # the same two vectors placed at positions (3, 1) and (9, 7): equal dot products after
    # rotation; at (3, 2) it differs
    d = 32
    a = _x(1, 1, d, seed=6)[0, 0]
    b = _x(1, 1, d, seed=7)[0, 0]
    L = 10
    cos, sin = make_rope_tables(L, d, base=100.0)
    cos, sin = cos.double().numpy(), sin.double().numpy()
    y = np.zeros((L, 1, d))
    y[:] = a
    ra = rope(y, cos, sin, interleaved)[:, 0]
    y[:] = b
    rb = rope(y, cos, sin, interleaved)[:, 0]
    assert abs(ra[3] @ rb[1] - ra[9] @ rb[7]) < 1e-5
    assert abs(ra[3] @ rb[1] - ra[3] @ rb[2]) > 1e-3


def test_interleaved_is_complex_multiplication():
    L, d = 5, 16
    y = _x(L, 2, d, seed=8)
    ang = np.random.default_rng(0).uniform(-3, 3, size=(L, d // 2))
    out = rope(y, np.cos(ang), np.sin(ang), interleaved=True)
    z = (y[..., 0::2] + 1j * y[..., 1::2]) * np.exp(1j * ang)[:, None, :]
    np.testing.assert_allclose(out[..., 0::2], z.real, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out[..., 1::2], z.imag, rtol=1e-12, atol=1e-14)


def test_conventions_differ_by_a_channel_permutation():
    L, d = 4, 16
    y = _x(L, 2, d, seed=9)
    ang = np.random.default_rng(1).uniform(-3, 3, size=(L, d // 2))
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # interleaved -> halves
    half = rope(y[..., perm], np.cos(ang), np.sin(ang), interleaved=False)
    inter = rope(y, np.cos(ang), np.sin(ang), interleaved=True)
    np.testing.assert_allclose(inter[..., perm], half, rtol=1e-13, atol=1e-14)


def test_reference_is_norm_then_rope_per_tensor():
    L, H, d = 7, 3, 64
    q, k = _x(L, H, d, seed=10, scale=2.0), _x(L, H, d, seed=11, scale=0.5)
    wq, wk = np.linspace(0.8, 1.2, d), np.linspace(1.1, 0.9, d)
    cos, sin = make_rope_tables(L, d)
    qo, ko = qk_norm_rope_reference(q, k, cos, sin, wq, wk, eps=1e-5)
    # by hand for one element of each: channel 3 (pair 3, first half) of row 5, head 1
    for x, w, o in ((q, wq, qo), (k, wk, ko)):
        v = x[5, 1]
        n = v / math.sqrt(np.mean(v * v) + 1e-5) * w
        c, s = float(cos[5, 3]), float(sin[5, 3])
        assert abs(o[5, 1, 3] - (n[3] * c - n[3 + d // 2] * s)) < 1e-12
        assert abs(o[5, 1, 3 + d // 2] - (n[3 + d // 2] * c + n[3] * s)) < 1e-12
