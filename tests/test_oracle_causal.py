"""Pins of the causal-attention oracle (CPU only).

The oracle is checked against things other than itself: a pure-Python brute force on tiny
inputs, torch's float64 causal scaled-dot-product attention (the routine the audio VAE
calls by default), the window oracle's masked dense attention with a lower-triangular mask,
and closed forms (the first row copies v_0; equal keys average v_0..v_i).
"""

import math

import numpy as np
import pytest
import torch

from oracle import (
    causal_attention_reference,
    causal_attention_rows,
    causal_mask,
    causal_pairs_per_head,
    masked_dense_attention,
)


def _inputs(n, H, d, seed=0, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return tuple(torch.randn(n, H, d, generator=g, dtype=torch.float64).to(dtype) for _ in range(3))


def _brute(q, k, v):
    n, H, d = q.shape
    out = np.zeros((n, H, d))
    for h in range(H):
        for i in range(n):
            s = [sum(q[i, h, c] * k[j, h, c] for c in range(d)) / math.sqrt(d) for j in range(i + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for c in range(d):
                out[i, h, c] = sum(w[j] * v[j, h, c] for j in range(i + 1)) / z
    return out


def test_brute_force_tiny():
    q, k, v = (x.numpy() for x in _inputs(7, 2, 4, seed=3))
    np.testing.assert_allclose(causal_attention_reference(q, k, v, block=3), _brute(q, k, v), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n,H,d,block", [(1, 1, 8, 4), (33, 2, 16, 8), (130, 3, 64, 64), (257, 1, 128, 256)])
def test_matches_torch_causal_sdpa_fp64(n, H, d, block):
    q, k, v = _inputs(n, H, d, seed=n)
    want = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True).transpose(0, 1)
    got = causal_attention_reference(q, k, v, block=block)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)


def test_matches_masked_dense_with_lower_triangle():
    q, k, v = _inputs(45, 2, 32, seed=9)
    got = causal_attention_reference(q, k, v, block=16)
    want = masked_dense_attention(q, k, v, causal_mask(45))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_rows_helper_matches_full():
    q, k, v = _inputs(70, 3, 16, seed=5)
    full = causal_attention_reference(q, k, v, block=32)
    rows, heads = [0, 1, 31, 32, 69], [2, 0]
    np.testing.assert_allclose(causal_attention_rows(q, k, v, rows, heads), full[rows][:, heads], rtol=1e-12, atol=1e-13)


def test_first_row_copies_v0_and_equal_keys_average():
    q, k, v = _inputs(20, 2, 8, seed=1)
    out = causal_attention_reference(q, k, v, block=8)
    np.testing.assert_allclose(out[0], v[0].numpy(), rtol=0, atol=1e-15)
    k_eq = k[:1].expand(20, 2, 8).contiguous()
    out = causal_attention_reference(q, k_eq, v, block=8)
    means = np.cumsum(v.numpy(), axis=0) / np.arange(1, 21)[:, None, None]
    np.testing.assert_allclose(out, means, rtol=1e-12, atol=1e-13)


def test_pairs_and_mask():
    assert causal_pairs_per_head(1) == 1 and causal_pairs_per_head(4096) == 4096 * 4097 // 2
    m = causal_mask(5)
    assert m.sum() == causal_pairs_per_head(5) and m[4, 0] and not m[0, 4]


def test_later_keys_do_not_matter():
    q, k, v = _inputs(40, 1, 16, seed=2)
    a = causal_attention_reference(q, k, v, block=16)
    k2, v2 = k.clone(), v.clone()
    k2[30:] += 5.0
    v2[30:] -= 3.0
    b = causal_attention_reference(q, k2, v2, block=16)
    np.testing.assert_array_equal(a[:30], b[:30])
    assert np.abs(a[30:] - b[30:]).max() > 1e-3
