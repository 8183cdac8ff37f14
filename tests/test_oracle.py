"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

* Equivalence of the decomposed (per-frame, window-bounds) form with brute-force
  explicitly masked attention whose mask is built pairwise from chunk distance
  (VDN-Minimax-H3 window-attention article, §三: the two forms are mathematically
  equal).
* Reductions to textbook SDPA (torch's float64 CPU implementation): radius covering
  every chunk, block-diagonal per-frame attention, and the global rows.
* Invariants: rows of the softmax sum to one, within-frame permutation
  equivariance, locality of the window, time reversal.
* Plans: hand-derived golden plans, brute-force grouping by identical mask rows, a
  closed-form group count and a chunk-pair count of kept pairs.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    Geometry,
    kept_pairs_per_head,
    masked_dense_attention,
    plan_groups,
    plan_kv_indices,
    window_attention_reference,
    window_attention_rows,
    window_mask,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(L, H, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((L, H, d)) for _ in range(3))


def _sdpa64(q, k, v):
    """torch SDPA in float64 on [L, H, d] arrays (default scale 1/sqrt(d))."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    return o[0].permute(1, 0, 2).numpy()


# ------------------------------------------------------------------ values vs brute force


SMALL_GEOMS = [
    Geometry(T, S, G, K, r)
    for T, S, G, K, r in itertools.product(range(1, 9), (1, 3), (0, 2), (1, 2, 3, 4), (0, 1, 2, 4))
]


@pytest.mark.parametrize("geom", SMALL_GEOMS, ids=lambda g: f"T{g.T}S{g.S}G{g.G}K{g.K}r{g.radius}")
def test_reference_equals_masked_dense(geom):
    q, k, v = _rand(geom.L, 2, 8, seed=geom.T * 1000 + geom.S * 100 + geom.K * 10 + geom.radius)
    ref = window_attention_reference(q, k, v, geom)
    brute = masked_dense_attention(q, k, v, window_mask(geom))
    np.testing.assert_allclose(ref, brute, rtol=0, atol=1e-12)


def test_rows_helper_equals_reference():
    geom = Geometry(7, 5, 3, 2, 1)
    q, k, v = _rand(geom.L, 3, 16, seed=5)
    ref = window_attention_reference(q, k, v, geom)
    rows = [0, 4, 9, 17, 34, 35, 36, 37]
    heads = [0, 2]
    got = window_attention_rows(q, k, v, geom, rows, heads)
    np.testing.assert_allclose(got, ref[rows][:, heads], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ reductions to SDPA


@pytest.mark.parametrize("T,S,G,K", [(8, 4, 0, 1), (8, 4, 3, 2), (5, 6, 2, 4), (3, 7, 0, 3)])
def test_radius_covering_all_chunks_is_full_attention(T, S, G, K):
    C = -(-T // K)
    for r in (C - 1, C, C + 3):
        geom = Geometry(T, S, G, K, r)
        q, k, v = _rand(geom.L, 2, 16, seed=T + S + G + K + r)
        np.testing.assert_allclose(window_attention_reference(q, k, v, geom), _sdpa64(q, k, v), rtol=0, atol=1e-12)


def test_block_diagonal_per_frame():
    geom = Geometry(T=6, S=5, G=0, K=1, radius=0)
    q, k, v = _rand(geom.L, 2, 16, seed=11)
    ref = window_attention_reference(q, k, v, geom)
    for t in range(geom.T):
        rows = slice(t * geom.S, (t + 1) * geom.S)
        np.testing.assert_allclose(ref[rows], _sdpa64(q[rows], k[rows], v[rows]), rtol=0, atol=1e-12)


def test_global_rows_are_full_attention_rows():
    geom = Geometry(T=9, S=4, G=5, K=2, radius=1)
    q, k, v = _rand(geom.L, 2, 16, seed=12)
    ref = window_attention_reference(q, k, v, geom)
    full = _sdpa64(q, k, v)
    np.testing.assert_allclose(ref[geom.n_frame_rows:], full[geom.n_frame_rows:], rtol=0, atol=1e-12)
    # and frame rows are not (the window actually removes keys here)
    assert np.abs(ref[: geom.n_frame_rows] - full[: geom.n_frame_rows]).max() > 1e-3


# ------------------------------------------------------------------ invariants


def test_rows_sum_to_one():
    geom = Geometry(T=10, S=3, G=4, K=3, radius=1)
    q, k, _ = _rand(geom.L, 2, 16, seed=3)
    out = window_attention_reference(q, k, np.ones_like(q), geom)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)


def test_within_frame_permutation_equivariance():
    geom = Geometry(T=7, S=6, G=3, K=2, radius=1)
    q, k, v = _rand(geom.L, 2, 16, seed=4)
    rng = np.random.default_rng(0)
    perm = np.arange(geom.L)
    for t in range(geom.T):
        perm[t * geom.S:(t + 1) * geom.S] = t * geom.S + rng.permutation(geom.S)
    perm[geom.n_frame_rows:] = geom.n_frame_rows + rng.permutation(geom.G)
    out = window_attention_reference(q, k, v, geom)
    out_p = window_attention_reference(q[perm], k[perm], v[perm], geom)
    np.testing.assert_allclose(out_p, out[perm], rtol=0, atol=1e-12)


def test_locality_outside_window_is_ignored():
    geom = Geometry(T=12, S=3, G=2, K=2, radius=1)
    q, k, v = _rand(geom.L, 1, 8, seed=8)
    base = window_attention_reference(q, k, v, geom)
    # frame 0 (chunk 0) sees chunks 0..1 = frames 0..3 = rows [0, 12) plus globals
    k2, v2 = k.copy(), v.copy()
    k2[12:geom.n_frame_rows] += 5.0
    v2[12:geom.n_frame_rows] -= 3.0
    pert = window_attention_reference(q, k2, v2, geom)
    np.testing.assert_array_equal(pert[:6], base[:6])       # chunk 0 rows: untouched
    assert np.abs(pert[6:12] - base[6:12]).max() > 1e-3      # chunk 1 sees chunk 2: changed
    assert np.abs(pert[geom.n_frame_rows:] - base[geom.n_frame_rows:]).max() > 1e-3  # globals see all


def test_time_reversal():
    geom = Geometry(T=12, S=4, G=3, K=3, radius=1)
    q, k, v = _rand(geom.L, 2, 8, seed=9)
    rev = np.concatenate([
        np.concatenate([np.arange(t * geom.S, (t + 1) * geom.S) for t in reversed(range(geom.T))]),
        np.arange(geom.n_frame_rows, geom.L),
    ])
    out = window_attention_reference(q, k, v, geom)
    out_r = window_attention_reference(q[rev], k[rev], v[rev], geom)
    np.testing.assert_allclose(out_r, out[rev], rtol=0, atol=1e-12)


def test_plausible_mistakes_are_caught():
    """A wrong window (off by one chunk) must disagree with the reference."""
    geom = Geometry(T=9, S=3, G=2, K=2, radius=1)
    q, k, v = _rand(geom.L, 1, 8, seed=10)
    ref = window_attention_reference(q, k, v, geom)
    for wrong in (Geometry(9, 3, 2, 2, 0), Geometry(9, 3, 2, 2, 2), Geometry(9, 3, 2, 3, 1)):
        assert np.abs(masked_dense_attention(q, k, v, window_mask(wrong)) - ref).max() > 1e-3


# ------------------------------------------------------------------ plans


def _read_golden(name):
    geom, groups, glob, pairs = None, [], None, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if not line:
                continue
            vals = [int(x) for x in line[1:]]
            if line[0] == "geometry":
                geom = Geometry(*vals)
            elif line[0] == "group":
                groups.append(tuple(vals))
            elif line[0] == "global":
                glob = tuple(vals)
            elif line[0] == "kept_pairs_per_head":
                pairs = vals[0]
    return geom, groups, glob, pairs


@pytest.mark.parametrize("name", ["tiny_plan.txt", "ragged_plan.txt"])
def test_plan_matches_hand_derived_golden(name):
    geom, groups, glob, pairs = _read_golden(name)
    got = [(g.q_begin, g.q_end, g.kv_begin, g.kv_end, g.chunk_lo, g.chunk_hi) for g in plan_groups(geom)]
    assert got == groups
    assert glob == (geom.n_frame_rows, geom.L, 0, geom.L)
    if pairs is not None:
        assert kept_pairs_per_head(geom) == pairs


def _closed_form_groups(C, r):
    n_full = min(r, C - 1) - max(0, C - 1 - r) + 1
    return C if n_full <= 1 else C - n_full + 1


def _kept_pairs_chunk_pairs(geom):
    """Kept pairs counted over pairs of chunks at distance <= radius, plus globals."""
    rows = [(min(geom.T, (c + 1) * geom.K) - c * geom.K) * geom.S for c in range(geom.n_chunks)]
    frame = sum(rows[a] * rows[b] for a in range(geom.n_chunks) for b in range(geom.n_chunks)
                if abs(a - b) <= geom.radius)
    n = geom.n_frame_rows
    return frame + 2 * geom.G * n + geom.G * geom.G


@pytest.mark.parametrize("T,S,G,K,r", list(itertools.product(range(1, 14), (1, 2, 3), (0, 3), range(1, 6), range(0, 8)))[::7])
def test_plan_brute_force_and_closed_forms(T, S, G, K, r):
    geom = Geometry(T, S, G, K, r)
    groups = plan_groups(geom)
    # closed-form count
    assert len(groups) == _closed_form_groups(geom.n_chunks, r)
    # groups partition the frame rows in order; adjacent groups differ (maximal)
    assert groups[0].q_begin == 0 and groups[-1].q_end == geom.n_frame_rows
    for a, b in zip(groups, groups[1:]):
        assert a.q_end == b.q_begin
        assert (a.kv_begin, a.kv_end) != (b.kv_begin, b.kv_end)
    # brute force: rows grouped by identical rows of the pairwise mask
    mask = window_mask(geom)
    for g in groups:
        want = plan_kv_indices(geom, g)
        for i in range(g.q_begin, g.q_end):
            np.testing.assert_array_equal(np.flatnonzero(mask[i]), want)
    # kept pairs: chunk-pair count and mask count
    assert kept_pairs_per_head(geom) == _kept_pairs_chunk_pairs(geom) == int(mask.sum())


@pytest.mark.parametrize("T,S,G,K,r,pairs", [
    (6, 16, 8, 2, 1, 8768),
    (24, 256, 256, 3, 1, 16187392),
    (102, 960, 1024, 3, 1, 1031028736),
    (50, 432, 77, 4, 2, 171293929),
    (8, 1024, 0, 1, 8, 67108864),
])
def test_kept_pairs_of_named_workloads(T, S, G, K, r, pairs):
    geom = Geometry(T, S, G, K, r)
    assert kept_pairs_per_head(geom) == pairs == _kept_pairs_chunk_pairs(geom)


def test_dense_workload_reduces_to_one_group():
    geom = Geometry(8, 1024, 0, 1, 8)
    groups = plan_groups(geom)
    assert len(groups) == 1 and (groups[0].kv_begin, groups[0].kv_end) == (0, geom.L)
