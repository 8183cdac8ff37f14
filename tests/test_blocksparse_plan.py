"""Host-side checks of the block-sparse plan (wa_blocksparse_plan_create): its block mask
bit for bit against the oracle's (the FlexAttention-style BlockMask of the frame rows,
[VDN] §二), its work items' tile lists against a construction from that mask, the global leg
identical to the decomposed plan's, the launch order, the computed-pair count, and the
status codes.  No GPU needed."""

import itertools

import numpy as np
import pytest

import chunk_windowed_softmax_amd as wa
from oracle import Geometry
from oracle.block_mask import block_mask

NAMED = {
    "tiny": (6, 16, 8, 2, 1, 1, 64),
    "small": (24, 256, 256, 3, 1, 8, 128),
    "h3": (102, 960, 1024, 3, 1, 7, 128),
    "ragged": (50, 432, 77, 4, 2, 16, 128),
    "dense": (8, 1024, 0, 1, 8, 16, 64),
}
BLOCKS = [(128, 64), (256, 128), (128, 128), (256, 64)]
TILE = 64
ITEM_ROWS = 256


@pytest.fixture(scope="module")
def lib():
    return wa.load_library()


def _expected_tiles(geom, bq, bk):
    """Per frame item (256 rows = 256 / bq query blocks): [(first key, needs_mask)], from the
    oracle's block mask."""
    kv_num, kv_idx, full_num, full_idx = block_mask(geom, bq, bk)
    L = geom.L
    items = []
    per = ITEM_ROWS // bq
    for i0 in range(0, len(kv_num), per):
        listed, full_all = set(), None
        for i in range(i0, min(len(kv_num), i0 + per)):
            part = set(kv_idx[i, :kv_num[i]].tolist())
            full = set(full_idx[i, :full_num[i]].tolist())
            listed |= part | full
            full_all = full if full_all is None else full_all & full
        tiles = []
        for j in sorted(listed):
            k0, k1 = j * bk, min(L, (j + 1) * bk)
            for t0 in range(k0, k1, TILE):
                tiles.append((t0, int(j not in full_all or t0 + TILE > k1)))
        items.append(((i0 * bq, min(geom.n_frame_rows, (i0 + per) * bq)), tiles))
    return items


def _check(T, S, G, K, r, H, d, bq, bk):
    geom = Geometry(T, S, G, K, r)
    plan = wa.wa_blocksparse_plan_create(T, S, G, K, r, H, d, bq, bk)
    info = plan.info
    assert (info["block_q"], info["block_kv"]) == (bq, bk)
    got = wa.wa_plan_block_mask(plan)
    for a, b in zip(got, block_mask(geom, bq, bk)):
        np.testing.assert_array_equal(a, b)
    items = wa.wa_plan_items(plan)
    tiles = wa.wa_plan_tiles(plan)
    assert len(tiles) == info["n_tiles"]
    assert (items[:, wa.WA_ITEM_COLS - 1] == 2).all()  # every item is a tile list
    exp = _expected_tiles(geom, bq, bk)
    frame = items[: len(exp)]
    computed = 0
    for it, ((q0, q1), tl) in zip(frame, exp):
        assert (it[0], it[1]) == (q0, q1)
        ent = tiles[it[2]: it[2] + it[3]]
        assert [(int(e) >> 1, int(e) & 1) for e in ent] == tl
        computed += (q1 - q0) * len(tl) * TILE
    # global leg: the decomposed plan's key splits, as contiguous tile lists
    dec = wa.wa_plan_create(T, S, G, K, r, H, d)
    assert info["n_splits"] == dec.info["n_splits"]
    dec_items = wa.wa_plan_items(dec)
    dec_glob = dec_items[dec_items[:, 0] >= T * S]
    glob = items[len(exp):]
    assert len(glob) == len(dec_glob)
    L = geom.L
    for it, di in zip(glob, dec_glob):
        assert (it[0], it[1], it[6]) == (di[0], di[1], di[6])
        ent = tiles[it[2]: it[2] + it[3]]
        starts = [int(e) >> 1 for e in ent]
        assert starts == list(range(di[2], di[3], TILE))
        assert [int(e) & 1 for e in ent] == [int(s + TILE > di[3]) for s in starts]
        computed += (it[1] - it[0]) * len(ent) * TILE
    assert info["computed_pairs_per_head"] == computed
    assert info["computed_pairs_per_head"] >= info["kept_pairs_per_head"]
    order = wa.wa_plan_launch_order(plan)
    assert sorted(order[order >= 0].tolist()) == list(range(H * info["n_items"]))
    return plan


@pytest.mark.parametrize("name", sorted(NAMED))
@pytest.mark.parametrize("bq,bk", BLOCKS[:2])
def test_named_geometries(lib, name, bq, bk):
    _check(*NAMED[name], bq, bk)


def test_sweep(lib):
    for (T, S, G, K, r), (bq, bk) in itertools.product(
            itertools.product((1, 3, 7, 13), (1, 50, 130), (0, 3, 70), (1, 2, 5), (0, 1, 4)), BLOCKS):
        _check(T, S, G, K, r, 2, 64, bq, bk)


def test_block_sizes_and_limits(lib):
    with pytest.raises(wa.WaError) as e:
        wa.wa_blocksparse_plan_create(6, 16, 8, 2, 1, 1, 64, 64, 64)
    assert e.value.code == wa.WA_ERR_UNSUPPORTED
    with pytest.raises(wa.WaError) as e:
        wa.wa_blocksparse_plan_create(6, 16, 8, 2, 1, 1, 64, 256, 32)
    assert e.value.code == wa.WA_ERR_UNSUPPORTED
    with pytest.raises(wa.WaError) as e:
        wa.wa_blocksparse_plan_create(6, 16, 8, 2, 1, 1, 64, 0, 128)
    assert e.value.code == wa.WA_ERR_INVALID
    with pytest.raises(wa.WaError) as e:
        wa.wa_blocksparse_plan_create(0, 16, 8, 2, 1, 1, 64, 256, 128)
    assert e.value.code == wa.WA_ERR_INVALID
    # an item whose tile list would not fit the kernel's LDS list (every key kept)
    with pytest.raises(wa.WaError) as e:
        wa.wa_blocksparse_plan_create(600, 1000, 0, 1, 1000, 1, 64, 256, 128)
    assert e.value.code == wa.WA_ERR_UNSUPPORTED and "tiles" in str(e.value)
    # the block mask of a plan without one
    with pytest.raises(wa.WaError):
        wa.wa_plan_block_mask(wa.wa_plan_create(6, 16, 8, 2, 1, 1, 64))


def test_blocksparse_plans_are_cached_apart(lib):
    a = wa.wa_blocksparse_plan_create(24, 256, 256, 3, 1, 8, 128, 256, 128)
    b = wa.wa_blocksparse_plan_create(24, 256, 256, 3, 1, 8, 128, 256, 128)
    c = wa.wa_blocksparse_plan_create(24, 256, 256, 3, 1, 8, 128, 128, 64)
    d = wa.wa_plan_create(24, 256, 256, 3, 1, 8, 128)
    assert a.handle.value == b.handle.value
    assert len({a.handle.value, c.handle.value, d.handle.value}) == 3
    assert d.info["block_q"] == 0 and d.info["n_tiles"] == 0
