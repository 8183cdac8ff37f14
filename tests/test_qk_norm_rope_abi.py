"""Host-side checks of wa_qk_norm_rope's argument validation.  Every call here is rejected
(or, with L = 0, accepted) before anything reaches the device, so no GPU is needed; the
pointers are plain aligned integers that are never dereferenced."""

import ctypes

import pytest

import chunk_windowed_softmax_amd as wa

BASE = 1 << 32  # fake, 256-byte aligned addresses far apart


def _addr(i):
    return BASE + i * (1 << 28)


def _call(lib, L=4, H=2, d=128, eps=1e-6, flags=0, dtype=wa.WA_BF16, **ptrs):
    p = dict(q=_addr(0), k=_addr(1), q_out=_addr(2), k_out=_addr(3), cos=_addr(4), sin=_addr(5), wq=None, wk=None)
    p.update(ptrs)
    return lib.wa_qk_norm_rope(p["q"], p["k"], p["q_out"], p["k_out"], p["cos"], p["sin"], p["wq"], p["wk"],
                               L, H, d, eps, flags, dtype, None)


@pytest.fixture(scope="module")
def lib():
    return wa.load_library()


def test_empty_is_a_no_op(lib):
    assert _call(lib, L=0) == wa.WA_OK
    assert _call(lib, L=0, q_out=_addr(0), k_out=_addr(1)) == wa.WA_OK
    nulls = dict(q=None, k=None, q_out=None, k_out=None, cos=None, sin=None)
    assert _call(lib, L=0, **nulls) == wa.WA_OK  # an empty tensor may have no storage
    assert _call(lib, L=0, d=96) == wa.WA_ERR_UNSUPPORTED  # scalars are still checked


@pytest.mark.parametrize("name", ["q", "k", "q_out", "k_out", "cos", "sin"])
def test_null_tensor_rejected(lib, name):
    assert _call(lib, **{name: None}) == wa.WA_ERR_INVALID
    assert "NULL" in wa.wa_last_error()


@pytest.mark.parametrize("name", ["q", "k", "q_out", "k_out", "cos", "sin", "wq", "wk"])
def test_misaligned_rejected(lib, name):
    assert _call(lib, **{name: _addr(7) + 8}) == wa.WA_ERR_INVALID
    assert "aligned" in wa.wa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wa.WA_ERR_INVALID),
    (dict(flags=2), wa.WA_ERR_INVALID),
    (dict(L=-1), wa.WA_ERR_INVALID),
    (dict(H=0), wa.WA_ERR_INVALID),
    (dict(eps=-1e-6), wa.WA_ERR_INVALID),
    (dict(eps=float("nan")), wa.WA_ERR_INVALID),
    (dict(eps=float("inf")), wa.WA_ERR_INVALID),
    (dict(d=96), wa.WA_ERR_UNSUPPORTED),
    (dict(d=256), wa.WA_ERR_UNSUPPORTED),
    (dict(L=1 << 20, H=16, d=128), wa.WA_ERR_UNSUPPORTED),
])
def test_bad_arguments_rejected(lib, kw, code):
    assert _call(lib, **kw) == code
    assert wa.wa_last_error()


@pytest.mark.parametrize("ptrs", [
    dict(q_out=_addr(0) + 256),            # q_out starts inside q
    dict(q_out=_addr(1)),                  # q_out is k
    dict(k_out=_addr(0)),                  # k_out is q
    dict(k_out=_addr(2) + 512),            # k_out inside q_out
    dict(q_out=_addr(3)),                  # q_out is k_out
])
def test_overlaps_rejected(lib, ptrs):
    assert _call(lib, L=4, H=2, d=128, **ptrs) == wa.WA_ERR_INVALID
    assert "overlap" in wa.wa_last_error()


def test_symbol_is_exported(lib):
    assert "wa_qk_norm_rope" in wa.EXPORTED_SYMBOLS
    assert isinstance(lib.wa_qk_norm_rope, ctypes._CFuncPtr)
