"""Host-side checks of the C ABI: exports, plan tables bit for bit against the oracle's
independent plan, work-item coverage, status codes and the plan cache.  No GPU needed:
building a plan touches no device."""

import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import chunk_windowed_softmax_amd as wa
from oracle import Geometry, kept_pairs_per_head, plan_groups, plan_kv_indices

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NAMED = {
    "tiny": (6, 16, 8, 2, 1, 1, 64),
    "small": (24, 256, 256, 3, 1, 8, 128),
    "h3": (102, 960, 1024, 3, 1, 7, 128),
    "h3_full": (102, 960, 1024, 3, 1, 56, 128),
    "ragged": (50, 432, 77, 4, 2, 16, 128),
    "dense": (8, 1024, 0, 1, 8, 16, 64),
}


@pytest.fixture(scope="module")
def lib():
    return wa.load_library()


def test_header_declares_exactly_the_exported_symbols(lib):
    with open(os.path.join(ROOT, "include", "wa.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(wa_\w+)\s*\(", header, re.M))
    assert declared == set(wa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def _check_plan_against_oracle(T, S, G, K, r, H, d):
    plan = wa.wa_plan_create(T, S, G, K, r, H, d)
    geom = Geometry(T, S, G, K, r)
    ref = plan_groups(geom)
    got = wa.wa_plan_groups(plan)
    want = np.array([[g.q_begin, g.q_end, g.kv_begin, g.kv_end, g.chunk_lo, g.chunk_hi] for g in ref], dtype=np.int32)
    np.testing.assert_array_equal(got, want)
    for gi, g in enumerate(ref):
        np.testing.assert_array_equal(wa.wa_plan_kv_indices(plan, gi), plan_kv_indices(geom, g).astype(np.int32))
    info = plan.info
    assert info["kept_pairs_per_head"] == kept_pairs_per_head(geom)
    assert info["L"] == geom.L and info["n_chunks"] == geom.n_chunks and info["n_groups"] == len(ref)
    _check_items_cover(plan, geom)
    _check_launch_order(plan, H)
    return plan


def _check_launch_order(plan, H):
    """The launch order runs every (head, item) unit exactly once; per XCD queue the window
    units come first, in increasing order (a contiguous run), then the global-leg units, all
    packed at the front of the row (the kernel's queues stop at the first -1)."""
    info = plan.info
    order = wa.wa_plan_launch_order(plan)
    assert order.shape == (info["launch_xcds"], info["launch_per_xcd"])
    n_items = info["n_items"]
    items = wa.wa_plan_items(plan)
    n_window = int((items[:, 0] < info["T"] * info["S"]).sum())
    units = order[order >= 0]
    assert sorted(units.tolist()) == list(range(H * n_items))
    for queue in order:
        q = queue[queue >= 0]
        assert (queue[:len(q)] >= 0).all() and (queue[len(q):] == -1).all()
        is_win = (q % n_items) < n_window
        k = int(is_win.sum())
        assert is_win[:k].all() and not is_win[k:].any()
        if k:
            assert (np.diff(q[:k]) > 0).all()


def _check_items_cover(plan, geom):
    """Every frame row is in exactly one final window item whose keys are its kept set;
    every global row is covered by splits that partition [0, L)."""
    items = wa.wa_plan_items(plan)
    info = plan.info
    n = geom.n_frame_rows
    cover = np.zeros(geom.L, dtype=np.int64)
    split_keys = {}
    groups = plan_groups(geom)
    for it in items:
        q0, q1, a0, b0, a1, b1, split, _ = (int(x) for x in it)
        assert 0 <= q0 < q1 <= geom.L and q1 - q0 <= info["block_m"]
        assert 0 <= a0 < b0 <= geom.L and 0 <= a1 <= b1 <= geom.L
        if q0 < n:
            assert q1 <= n and split == -1
            g = next(g for g in groups if g.q_begin <= q0 < g.q_end)
            assert q1 <= g.q_end and (a0, b0) == (g.kv_begin, g.kv_end) and (a1, b1) == (n, geom.L)
            cover[q0:q1] += 1
        else:
            assert (a1, b1) == (0, 0)
            assert (split == -1) == (info["n_splits"] == 1)
            split_keys.setdefault((q0, q1), []).append((a0, b0))
            if split <= 0:
                cover[q0:q1] += 1
    assert (cover == 1).all()
    for (q0, q1), ranges in split_keys.items():
        ranges.sort()
        assert ranges[0][0] == 0 and ranges[-1][1] == geom.L
        assert all(x[1] == y[0] for x, y in zip(ranges, ranges[1:]))
        assert len(ranges) == info["n_splits"]
        assert all((b - a) % info["block_n"] == 0 for a, b in ranges[:-1])


@pytest.mark.parametrize("name", sorted(NAMED))
def test_named_plans_bit_for_bit(lib, name):
    _check_plan_against_oracle(*NAMED[name])


@pytest.mark.parametrize("T,S,G,K,r", list(itertools.product(range(1, 14), (1, 2, 3), (0, 3), range(1, 6), range(0, 8)))[::5])
def test_plan_sweep_bit_for_bit(lib, T, S, G, K, r):
    _check_plan_against_oracle(T, S, G, K, r, 2, 64)


@pytest.mark.parametrize("args,code", [
    ((0, 16, 8, 2, 1, 1, 64), wa.WA_ERR_INVALID),
    ((6, 0, 8, 2, 1, 1, 64), wa.WA_ERR_INVALID),
    ((6, 16, -1, 2, 1, 1, 64), wa.WA_ERR_INVALID),
    ((6, 16, 8, 0, 1, 1, 64), wa.WA_ERR_INVALID),
    ((6, 16, 8, 2, -1, 1, 64), wa.WA_ERR_INVALID),
    ((6, 16, 8, 2, 1, 0, 64), wa.WA_ERR_INVALID),
    ((6, 16, 8, 2, 1, 1, 96), wa.WA_ERR_UNSUPPORTED),
    ((6, 16, 8, 2, 1, 1, 32), wa.WA_ERR_UNSUPPORTED),
    ((1000, 1000, 0, 1, 1, 40, 128), wa.WA_ERR_UNSUPPORTED),  # L*H*d >= 2^31
])
def test_invalid_geometry_status(lib, args, code):
    with pytest.raises(wa.WaError) as e:
        wa.wa_plan_create(*args)
    assert e.value.code == code
    assert wa.wa_last_error() != ""


def test_null_arguments(lib):
    assert lib.wa_plan_create(6, 16, 8, 2, 1, 1, 64, None) == wa.WA_ERR_INVALID
    assert lib.wa_plan_release(None) == wa.WA_ERR_INVALID
    assert lib.wa_forward(None, 16, 16, 16, 16, 0, None) == wa.WA_ERR_INVALID
    plan = wa.wa_plan_create(6, 16, 8, 2, 1, 1, 64)
    # NULL / misaligned / overlapping pointers and bad dtype are rejected before any device work
    assert lib.wa_forward(plan.handle, None, 16, 16, 16, 0, None) == wa.WA_ERR_INVALID
    assert lib.wa_forward(plan.handle, 16, 16, 16, 18, 0, None) == wa.WA_ERR_INVALID
    assert lib.wa_forward(plan.handle, 16, 32, 48, 64, 7, None) == wa.WA_ERR_INVALID
    assert lib.wa_forward(plan.handle, 1 << 20, 2 << 20, 3 << 20, (1 << 20) + 64, 0, None) == wa.WA_ERR_INVALID
    small = (ctypes.c_int32 * 1)()
    assert lib.wa_plan_groups(plan.handle, small, 1) == wa.WA_ERR_INVALID
    assert lib.wa_plan_kv_indices(plan.handle, 99, small, 1) == wa.WA_ERR_INVALID
    assert lib.wa_plan_items(plan.handle, small, 1) == wa.WA_ERR_INVALID
    assert lib.wa_plan_launch_order(plan.handle, small, 0) == wa.WA_ERR_INVALID
    assert lib.wa_plan_launch_order(None, small, 1) == wa.WA_ERR_INVALID


def test_plan_cache_and_refcounts(lib):
    a = wa.wa_plan_create(9, 5, 3, 2, 1, 2, 64)
    b = wa.wa_plan_create(9, 5, 3, 2, 1, 2, 64)
    assert a.handle.value == b.handle.value  # cached
    # four other geometries evict the first one; outstanding handles stay valid
    others = [wa.wa_plan_create(9, 5, 3, 2, 1, 2 + i, 64) for i in range(1, 5)]
    c = wa.wa_plan_create(9, 5, 3, 2, 1, 2, 64)
    assert c.info["H"] == 2
    np.testing.assert_array_equal(wa.wa_plan_groups(a), wa.wa_plan_groups(c))
    assert a.info == c.info
    for p in (a, b, c, *others):
        p.release()


@pytest.mark.parametrize("n,H,d", [(1, 1, 64), (255, 2, 64), (256, 1, 128), (1000, 3, 64), (16384, 16, 64)])
def test_causal_plan(lib, n, H, d):
    """Causal plans: block_m-row items over keys [0, q_end) flagged causal, no groups, the
    causal pair count, a full launch order."""
    plan = wa.wa_causal_plan_create(n, H, d)
    info = plan.info
    assert info["causal"] == 1 and info["n_groups"] == 0 and info["L"] == n and info["n_splits"] == 0
    assert info["kept_pairs_per_head"] == n * (n + 1) // 2
    items = wa.wa_plan_items(plan)
    bm = info["block_m"]
    assert len(items) == (n + bm - 1) // bm
    for j, it in enumerate(items):
        q0, q1, a0, b0, a1, b1, split, flags = (int(x) for x in it)
        assert (q0, q1) == (j * bm, min(n, (j + 1) * bm))
        assert (a0, b0, a1, b1, split, flags) == (0, q1, 0, 0, -1, 1)
    assert len(wa.wa_plan_groups(plan)) == 0
    _check_launch_order(plan, H)
    # distinct from the window plan of the same shape, and cached
    assert wa.wa_plan_create(1, n, 0, 1, 0, H, d).info["causal"] == 0
    again = wa.wa_causal_plan_create(n, H, d)
    assert again.handle.value == plan.handle.value


@pytest.mark.parametrize("args,code", [
    ((0, 1, 64), wa.WA_ERR_INVALID), ((4, 0, 64), wa.WA_ERR_INVALID),
    ((4, 1, 96), wa.WA_ERR_UNSUPPORTED), ((1 << 20, 32, 128), wa.WA_ERR_UNSUPPORTED),
])
def test_causal_plan_errors(lib, args, code):
    with pytest.raises(wa.WaError) as e:
        wa.wa_causal_plan_create(*args)
    assert e.value.code == code
    assert lib.wa_causal_plan_create(4, 1, 64, None) == wa.WA_ERR_INVALID
