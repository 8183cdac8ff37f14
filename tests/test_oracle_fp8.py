"""Pins of the fp8 oracle (oracle/fp8.py): the e4m3 decoder against torch's own float8_e4m3fn
conversion and the format's closed-form values, and the FP8 attention oracle against
invariants that hold for any correct attention of the decoded inputs."""

import numpy as np
import pytest
import torch

from chunk_windowed_softmax_amd.workloads import WORKLOADS, make_fp8_inputs, quantize_e4m3
from oracle import (Geometry, decode_e4m3, fp8_causal_attention_reference, fp8_window_attention_reference,
                    fp8_window_attention_rows)


def test_decode_matches_torch_float8_e4m3fn_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert (np.isnan(ours) == nan).all()
    np.testing.assert_array_equal(ours[~nan], theirs[~nan])
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0x7E, 448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x3C, 1.5), (0xB8, -1.0), (0xFE, -448.0), (0x00, 0.0),
])
def test_decode_closed_forms(code, value):
    assert decode_e4m3(np.array([code], dtype=np.uint8))[0] == value


def test_decode_is_monotone_and_sign_symmetric():
    pos = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()
    neg = decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8))
    np.testing.assert_array_equal(neg, -pos)
    assert np.signbit(decode_e4m3(np.array([0x80], dtype=np.uint8))[0])


def test_quantizer_uses_the_full_range():
    x = torch.randn(1000) * 3
    codes, scale = quantize_e4m3(x)
    vals = decode_e4m3(codes) * scale
    assert np.abs(vals).max() == pytest.approx(float(x.abs().max()), rel=2 ** -4)
    assert np.abs(vals - x.double().numpy()).max() <= 2 ** -4 * float(x.abs().max())


def _small_case(seed=0):
    w = WORKLOADS["small"]
    return w, make_fp8_inputs(w, seed)


def test_attention_depends_on_the_score_scale_product_only():
    w, (q8, k8, v8, sq, sk, sv) = _small_case()
    geom = Geometry(*w.geometry)
    rows, heads = [0, 700, w.L - 1], [0, 5]
    a = fp8_window_attention_rows(q8, k8, v8, sq, sk, sv, geom, rows, heads)
    b = fp8_window_attention_rows(q8, k8, v8, sq * 4.0, sk / 4.0, sv, geom, rows, heads)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    c = fp8_window_attention_rows(q8, k8, v8, sq, sk, sv * 3.0, geom, rows, heads)
    np.testing.assert_allclose(c, 3.0 * a, rtol=1e-12, atol=1e-12)


def test_constant_values_give_the_value_scale():
    """Softmax weights sum to one: v codes all 1.0 give exactly scale_v everywhere."""
    w, (q8, k8, v8, sq, sk, sv) = _small_case(1)
    ones = torch.full_like(v8, 0x38)
    out = fp8_window_attention_rows(q8, k8, ones, sq, sk, 0.25, Geometry(*w.geometry), [0, 1, 5000], [0, 7])
    np.testing.assert_allclose(out, 0.25, rtol=1e-12)


def test_zero_queries_give_the_mean_of_the_kept_values():
    """q = 0: uniform weights, so each row is the plain mean of its kept value rows."""
    L, H, d = 40, 1, 128
    geom = Geometry(4, 8, 8, 2, 0)  # 4 frames of 8 rows, chunks of 2 frames, radius 0, 8 global
    g = torch.Generator().manual_seed(3)
    k8, sk = quantize_e4m3(torch.randn(L, H, d, generator=g))
    v8, sv = quantize_e4m3(torch.randn(L, H, d, generator=g))
    q8 = torch.zeros_like(k8)
    out = fp8_window_attention_reference(q8, k8, v8, 1.0, sk, sv, geom)
    vals = decode_e4m3(v8) * sv
    np.testing.assert_allclose(out[0, 0], vals[list(range(0, 16)) + list(range(32, 40)), 0].mean(0), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(out[35, 0], vals[:, 0].mean(0), rtol=1e-12, atol=1e-14)  # a global row sees all keys


def test_causal_first_row_is_its_own_value():
    g = torch.Generator().manual_seed(4)
    q8, sq = quantize_e4m3(torch.randn(20, 2, 128, generator=g))
    k8, sk = quantize_e4m3(torch.randn(20, 2, 128, generator=g))
    v8, sv = quantize_e4m3(torch.randn(20, 2, 128, generator=g))
    out = fp8_causal_attention_reference(q8, k8, v8, sq, sk, sv)
    np.testing.assert_allclose(out[0], decode_e4m3(v8[0]) * sv, rtol=1e-12)
