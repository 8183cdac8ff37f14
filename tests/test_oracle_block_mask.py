"""Pins of the block-mask oracle (oracle/block_mask.py): the frame rows' block mask at
(block_q, block_kv) granularity, in the layout of FlexAttention's BlockMask ([VDN] §二).

The counting form (kept pairs per block, frame by frame) is checked against the block
mask read off the explicit pairwise [L, L] mask on every small geometry of a sweep, with
block sizes that do and do not divide the rows, and against closed forms: radius >= chunk
count keeps every pair (every whole block full), radius 0 with K = 1 and G = 0 keeps the
frame-diagonal blocks only, and a block mask always covers every kept pair."""

import itertools

import numpy as np
import pytest

from oracle import Geometry, kept_pairs_per_head, window_mask
from oracle.block_mask import block_mask, block_mask_brute_force, block_sparse_computed_pairs

SWEEP = [(T, S, G, K, r) for T, S, G, K, r in itertools.product(range(1, 8), (1, 3, 4), (0, 2, 5), (1, 2, 3), (0, 1, 3))]
BLOCKS = [(2, 2), (3, 2), (4, 8), (8, 4), (5, 3)]


@pytest.mark.parametrize("bq,bk", BLOCKS)
def test_counting_equals_brute_force(bq, bk):
    for T, S, G, K, r in SWEEP:
        geom = Geometry(T, S, G, K, r)
        got = block_mask(geom, bq, bk)
        want = block_mask_brute_force(geom, bq, bk)
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b, err_msg=str((T, S, G, K, r, bq, bk)))


@pytest.mark.parametrize("bq,bk", BLOCKS)
def test_every_kept_pair_is_in_a_listed_block(bq, bk):
    for T, S, G, K, r in SWEEP[::7]:
        geom = Geometry(T, S, G, K, r)
        kv_num, kv_idx, full_num, full_idx = block_mask(geom, bq, bk)
        m = window_mask(geom)[: geom.n_frame_rows]
        listed = np.zeros_like(m)
        for i in range(len(kv_num)):
            for j in list(kv_idx[i, :kv_num[i]]) + list(full_idx[i, :full_num[i]]):
                listed[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk] = True
        assert not (m & ~listed).any()
        # full blocks hold kept pairs only
        for i in range(len(full_num)):
            for j in full_idx[i, :full_num[i]]:
                assert m[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk].all()


def test_radius_beyond_chunks_makes_whole_blocks_full():
    geom = Geometry(8, 1024, 0, 1, 8)  # the dense degenerate workload
    kv_num, kv_idx, full_num, full_idx = block_mask(geom, 256, 128)
    assert (kv_num == 0).all() and (full_num == 64).all()
    np.testing.assert_array_equal(full_idx, np.tile(np.arange(64), (32, 1)))
    # a sequence length that is not a multiple of the key block: the cut block is partial
    geom = Geometry(5, 100, 0, 1, 5)
    kv_num, kv_idx, full_num, full_idx = block_mask(geom, 128, 64)
    assert (kv_num == 1).all() and (kv_idx[:, 0] == 7).all() and (full_num == 7).all()


def test_block_diagonal_when_every_frame_is_alone():
    # K = 1, radius 0, no globals: frame t keeps itself only; with S a multiple of both
    # block sizes the mask is block diagonal and full
    geom = Geometry(6, 128, 0, 1, 0)
    kv_num, kv_idx, full_num, full_idx = block_mask(geom, 64, 128)
    assert (kv_num == 0).all() and (full_num == 1).all()
    np.testing.assert_array_equal(full_idx[:, 0], np.arange(12) // 2)


def test_computed_pairs_bound_the_kept_pairs():
    for T, S, G, K, r in SWEEP[::5]:
        geom = Geometry(T, S, G, K, r)
        window_kept = kept_pairs_per_head(geom) - G * geom.L
        for bq, bk in BLOCKS:
            c = block_sparse_computed_pairs(geom, bq, bk)
            assert window_kept <= c <= geom.n_frame_rows * (-(-geom.L // bk)) * bk
    # blocks of one row and one key compute exactly the kept pairs
    geom = Geometry(5, 3, 2, 2, 1)
    assert block_sparse_computed_pairs(geom, 1, 1) == kept_pairs_per_head(geom) - 2 * geom.L
