"""GPU parity of the FP8 (e4m3) attention path (wa_forward_fp8) against the fp64 oracle of
the decoded inputs.

Tolerance.  Scores and the softmax run in fp32 on exact fp8 products; the one approximation
is rounding each softmax weight P <= 1 to e4m3 for the second product.  RNE to 3 mantissa
bits leaves a relative error of at most 2^-4 per weight, roughly uniform, so about 2.5-3.5%
RMS; the output is a weighted mean of value rows whose weights carry that error, so its
relative L2 error is of the same size (2.4-2.7% when the rounding is emulated on these
inputs).  Bound: relative L2 <= 4e-2, and per element |err| <= 2^-4 * max|v| (each weight
off by at most 2^-4 of itself, weights summing to one).  Cases whose weights are exactly
representable (q = 0: every weight 1; q = k at a large scale: one weight 1, the rest far
below e4m3's smallest subnormal) must match to bf16 rounding: |err| <= 2^-8 |ref| + 1e-3.
"""

import sys

import numpy as np
import pytest
import torch

from chunk_windowed_softmax_amd.workloads import WORKLOADS, make_fp8_inputs, quantize_e4m3
from oracle import (Geometry, decode_e4m3, fp8_causal_attention_reference, fp8_window_attention_reference,
                    fp8_window_attention_rows)

pytestmark = pytest.mark.gpu

REL_L2 = 4e-2


def _say(msg):
    print(f"[gpu-fp8] {msg}", flush=True)
    sys.stdout.flush()


def _check(got, ref, vmax, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _say(f"{what}: rel_l2={rel:.3e} max_abs={err.max():.3e} (bound {2 ** -4 * vmax:.3e})")
    assert np.isfinite(got).all()
    assert rel <= REL_L2, what
    assert err.max() <= 2 ** -4 * vmax, what


def _check_exact(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    worst = float((err / (2 ** -8 * np.abs(ref) + 1e-3)).max())
    _say(f"{what}: max_abs={err.max():.3e} worst err/bound={worst:.3f}")
    assert worst <= 1.0, what


def _plan(wa, w, H=None):
    return wa.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, H or w.H, w.d)


def _run(wa, plan, q8, k8, v8, sq, sk, sv):
    out = wa.wa_forward_fp8(plan, q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def test_fp8_full_parity_small(gpu_lib):
    w = WORKLOADS["small"]
    _say(f"small: T={w.T} S={w.S} G={w.G} K={w.K} r={w.radius} H={w.H}")
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(w, seed=0)
    got = _run(gpu_lib, _plan(gpu_lib, w), q8, k8, v8, sq, sk, sv)
    ref = fp8_window_attention_reference(q8, k8, v8, sq, sk, sv, Geometry(*w.geometry))
    _check(got, ref, np.nanmax(np.abs(decode_e4m3(v8))) * sv, "small")


@pytest.mark.parametrize("name", ["ragged", "h3", "h3_full"])
def test_fp8_sampled_parity(gpu_lib, name):
    """Sampled rows (first, last, frame and group edges, global rows, random) of every head;
    h3_full is the whole model's 56 heads on one GPU (the largest tensors, 709 MB each)."""
    w = WORKLOADS[name]
    _say(f"{name}: T={w.T} S={w.S} G={w.G} K={w.K} r={w.radius} H={w.H} (sampled rows)")
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(w, seed=1)
    got = _run(gpu_lib, _plan(gpu_lib, w), q8, k8, v8, sq, sk, sv)
    rng = np.random.default_rng(5)
    rows = {0, 1, w.L - 1, w.T * w.S - 1, w.T * w.S, w.S - 1, w.S, w.K * w.S - 1, w.K * w.S}
    rows |= set(rng.integers(0, w.L, 120).tolist())
    rows = sorted(r for r in rows if 0 <= r < w.L)
    ref = fp8_window_attention_rows(q8, k8, v8, sq, sk, sv, Geometry(*w.geometry), rows, list(range(w.H)))
    _check(got[rows], ref, np.nanmax(np.abs(decode_e4m3(v8))) * sv, name)


def test_fp8_causal_parity(gpu_lib):
    n, H, d = 1000, 2, 128
    g = torch.Generator().manual_seed(2)
    (q8, sq), (k8, sk), (v8, sv) = (quantize_e4m3(torch.randn(n, H, d, generator=g)) for _ in range(3))
    plan = gpu_lib.wa_causal_plan_create(n, H, d)
    got = _run(gpu_lib, plan, q8, k8, v8, sq, sk, sv)
    ref = fp8_causal_attention_reference(q8, k8, v8, sq, sk, sv)
    _check(got, ref, np.nanmax(np.abs(decode_e4m3(v8))) * sv, "causal 1000x2")


def test_fp8_zero_queries_exact(gpu_lib):
    """q = 0: every weight is exactly 1, so each row is the mean of its kept value rows."""
    w = WORKLOADS["small"]
    _, k8, v8, _, sk, sv = make_fp8_inputs(w, seed=3)
    q8 = torch.zeros_like(k8)
    got = _run(gpu_lib, _plan(gpu_lib, w), q8, k8, v8, 1.0, sk, sv)
    rows = [0, 255, 256, 3000, w.T * w.S - 1, w.T * w.S, w.L - 1]
    ref = fp8_window_attention_rows(q8, k8, v8, 1.0, sk, sv, Geometry(*w.geometry), rows, list(range(w.H)))
    _check_exact(got[rows], ref, "zero queries")


def test_fp8_self_attention_exact(gpu_lib):
    """q = k at a large scale: each row's own key outscores every other by 2^30 and more, so
    its weight is 1 and the others vanish below e4m3's range: the output is the row's value."""
    w = WORKLOADS["small"]
    g = torch.Generator().manual_seed(4)
    k8, sk = quantize_e4m3(torch.randn(w.L, w.H, w.d, generator=g) * 2.5)
    v8, sv = quantize_e4m3(torch.randn(w.L, w.H, w.d, generator=g))
    got = _run(gpu_lib, _plan(gpu_lib, w), k8, k8, v8, sk, sk, sv)
    rows = list(range(0, w.L, 97)) + [w.L - 1]
    ref = fp8_window_attention_rows(k8, k8, v8, sk, sk, sv, Geometry(*w.geometry), rows, list(range(w.H)))
    np.testing.assert_allclose(ref, decode_e4m3(v8[rows]) * sv, rtol=1e-6, atol=1e-6)  # the premise
    _check_exact(got[rows], ref, "self attention")


def test_fp8_rejects_other_head_sizes(gpu_lib):
    plan = gpu_lib.wa_plan_create(4, 16, 8, 2, 1, 1, 64)
    x = torch.zeros(72, 1, 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.WaError) as e:
        gpu_lib.wa_forward_fp8(plan, x, x, x, 1.0, 1.0, 1.0)
    assert e.value.code == 2


@pytest.mark.parametrize("geom,H", [((6, 300, 40, 1, 1), 2), ((7, 60, 33, 1, 2), 3), ((3, 64, 0, 2, 1), 1)])
def test_fp8_edge_geometries(gpu_lib, geom, H):
    """Ragged chunks and frames, items of one wave or less, no global rows: full comparison."""
    T, S, G, K, r = geom
    L = T * S + G
    g = torch.Generator().manual_seed(sum(geom) + H)
    (q8, sq), (k8, sk), (v8, sv) = (quantize_e4m3(torch.randn(L, H, 128, generator=g)) for _ in range(3))
    plan = gpu_lib.wa_plan_create(T, S, G, K, r, H, 128)
    got = _run(gpu_lib, plan, q8, k8, v8, sq, sk, sv)
    ref = fp8_window_attention_reference(q8, k8, v8, sq, sk, sv, Geometry(T, S, G, K, r))
    _check(got, ref, np.nanmax(np.abs(decode_e4m3(v8))) * sv, f"edge {geom} H={H}")


def test_fp8_short_items(gpu_lib):
    """Items of at most 64 rows (three 300-row groups ending in 44-row items, a 30-row
    global item) run split over the four waves by key half and merge the halves at the end.
    Full comparison on random inputs; constant value rows exact (the merged row sum must be
    the sum of exactly the rounded weights of both halves); q = k at a large scale exact
    (each row's own key sits in one half, far above everything in the other)."""
    T, S, G, K, r, H = 9, 100, 30, 3, 1, 2
    geom = Geometry(T, S, G, K, r)
    L = T * S + G
    plan = gpu_lib.wa_plan_create(T, S, G, K, r, H, 128)
    g = torch.Generator().manual_seed(12)
    (q8, sq), (k8, sk), (v8, sv) = (quantize_e4m3(torch.randn(L, H, 128, generator=g)) for _ in range(3))
    got = _run(gpu_lib, plan, q8, k8, v8, sq, sk, sv)
    ref = fp8_window_attention_reference(q8, k8, v8, sq, sk, sv, geom)
    _check(got, ref, np.nanmax(np.abs(decode_e4m3(v8))) * sv, "short items")
    row, svc = quantize_e4m3(torch.randn(1, 1, 128, generator=g))
    vc = row.expand(L, H, 128).contiguous()
    got = _run(gpu_lib, plan, q8, k8, vc, sq, sk, svc)
    _check_exact(got, np.broadcast_to(decode_e4m3(row) * svc, got.shape), "short items, constant values")
    k8, sk = quantize_e4m3(torch.randn(L, H, 128, generator=g) * 2.5)
    got = _run(gpu_lib, plan, k8, k8, v8, sk, sk, sv)
    rows = [0, 255, 256, 299, 300, 599, 856, 899, T * S, L - 1]
    ref = fp8_window_attention_rows(k8, k8, v8, sk, sk, sv, geom, rows, list(range(H)))
    np.testing.assert_allclose(ref, decode_e4m3(v8[rows]) * sv, rtol=1e-6, atol=1e-6)  # the premise
    _check_exact(got[rows], ref, "short items, self attention")


def test_fp8_covers_every_row_and_is_deterministic(gpu_lib):
    """Every output element is written (NaN prefill), and two calls agree bit for bit."""
    w = WORKLOADS["ragged"]
    q8, k8, v8, sq, sk, sv = (x.cuda() if torch.is_tensor(x) else x for x in make_fp8_inputs(w, seed=6))
    plan = _plan(gpu_lib, w)
    out = torch.full((w.L, w.H, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.wa_forward_fp8(plan, q8, k8, v8, sq, sk, sv, out=out)
    again = gpu_lib.wa_forward_fp8(plan, q8, k8, v8, sq, sk, sv)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    assert torch.equal(out, again)


def test_fp8_constant_values_exact(gpu_lib):
    """Every value row the same vector: whatever the weights, the output is that vector,
    provided each row is normalised by the sum of exactly the (e4m3-rounded) weights that
    multiply V.  Normalising by the unrounded sum would leave the rounding's relative error
    (up to 2^-4 per weight) in the output.  Random q and k at a wide score range, so many
    weights are far from representable, and the persistent launch of the ragged workload."""
    w = WORKLOADS["ragged"]
    g = torch.Generator().manual_seed(7)
    q8, sq = quantize_e4m3(torch.randn(w.L, w.H, w.d, generator=g) * 3.0)
    k8, sk = quantize_e4m3(torch.randn(w.L, w.H, w.d, generator=g) * 3.0)
    row, sv = quantize_e4m3(torch.randn(1, 1, w.d, generator=g))
    v8 = row.expand(w.L, w.H, w.d).contiguous()
    got = _run(gpu_lib, _plan(gpu_lib, w), q8, k8, v8, sq, sk, sv)
    want = np.broadcast_to(decode_e4m3(row) * sv, got.shape)
    _check_exact(got, want, "constant values")
