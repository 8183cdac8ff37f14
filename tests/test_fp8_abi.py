"""Host-side checks of wa_forward_fp8's argument validation: every call here is rejected
before anything reaches the device, so no GPU is needed (pointers are never dereferenced)."""

import pytest

import chunk_windowed_softmax_amd as wa

BASE = 1 << 32


def _addr(i):
    return BASE + i * (1 << 28)


@pytest.fixture(scope="module")
def plan():
    return wa.wa_plan_create(4, 16, 8, 2, 1, 2, 128)  # L = 72 rows, 2 heads, d = 128


def _call(plan, q=_addr(0), k=_addr(1), v=_addr(2), out=_addr(3), sq=1.0, sk=1.0, sv=1.0, handle=True):
    lib = wa.load_library()
    return lib.wa_forward_fp8(plan.handle if handle else None, q, k, v, sq, sk, sv, out, None)


def test_null_plan_and_tensors(plan):
    assert _call(plan, handle=False) == wa.WA_ERR_INVALID
    for name in ("q", "k", "v", "out"):
        assert _call(plan, **{name: None}) == wa.WA_ERR_INVALID


@pytest.mark.parametrize("name", ["q", "k", "v", "out"])
def test_misaligned(plan, name):
    assert _call(plan, **{name: _addr(5) + 4}) == wa.WA_ERR_INVALID
    assert "aligned" in wa.wa_last_error()


@pytest.mark.parametrize("scales", [(0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("nan")),
                                    (float("inf"), 1.0, 1.0)])
def test_bad_scales(plan, scales):
    sq, sk, sv = scales
    assert _call(plan, sq=sq, sk=sk, sv=sv) == wa.WA_ERR_INVALID
    assert "scale" in wa.wa_last_error()


def test_out_overlapping_an_input(plan):
    n = 72 * 2 * 128  # elements; inputs hold 1 byte each, out 2
    assert _call(plan, out=_addr(0) + 64) == wa.WA_ERR_INVALID        # out starts inside q
    assert _call(plan, q=_addr(3) + 2 * n - 16) == wa.WA_ERR_INVALID  # q starts inside out
    assert "overlap" in wa.wa_last_error()


def test_other_head_sizes_are_unsupported():
    p64 = wa.wa_plan_create(4, 16, 8, 2, 1, 1, 64)
    assert _call(p64) == wa.WA_ERR_UNSUPPORTED
