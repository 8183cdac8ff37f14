"""Chunk-windowed softmax attention for MI355X (gfx950): thin Python binding.

The work happens in ``libwa.so`` (HIP kernels behind the C ABI of ``include/wa.h``);
this module only marshals arguments.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is missing the calls raise.

Functions carry the C names:

* ``wa_plan_create(T, S, G, K, radius, H, d) -> Plan``
* ``wa_causal_plan_create(n, H, d) -> Plan`` (causal dense attention, the audio VAE's)
* ``wa_blocksparse_plan_create(T, S, G, K, radius, H, d, block_q, block_kv) -> Plan`` (block-sparse form)
* ``wa_forward(plan, q, k, v, out=None) -> out``
* ``wa_forward_noalloc(plan, q, k, v, out) -> out`` (same call; allocates nothing)
* ``wa_forward_fp8(plan, q8, k8, v8, scale_q, scale_k, scale_v, out=None) -> out`` (e4m3 inputs)
* ``wa_qk_norm_rope(q, k, cos, sin, wq=None, wk=None, ...) -> (q_out, k_out)`` (the prologue)
* ``wa_plan_info / wa_plan_groups / wa_plan_kv_indices / wa_plan_items / wa_plan_launch_order /
  wa_last_error``
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwa.so")

WA_OK, WA_ERR_INVALID, WA_ERR_UNSUPPORTED, WA_ERR_ALLOC, WA_ERR_HIP = range(5)
WA_BF16, WA_F32 = 0, 1
WA_ROPE_INTERLEAVED = 1
WA_ITEM_COLS = 8

# Every symbol include/wa.h declares.
EXPORTED_SYMBOLS = (
    "wa_plan_create",
    "wa_causal_plan_create",
    "wa_blocksparse_plan_create",
    "wa_plan_block_mask",
    "wa_plan_tiles",
    "wa_plan_release",
    "wa_forward",
    "wa_plan_info",
    "wa_plan_groups",
    "wa_plan_kv_indices",
    "wa_plan_items",
    "wa_plan_launch_order",
    "wa_qk_norm_rope",
    "wa_forward_fp8",
    "wa_forward_noalloc",
    "wa_last_error",
)


class WaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[wa status {code}] {msg}")
        self.code = code


class _PlanInfo(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("S", ctypes.c_int32), ("G", ctypes.c_int32), ("K", ctypes.c_int32),
        ("radius", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("L", ctypes.c_int32),
        ("n_chunks", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("kept_pairs_per_head", ctypes.c_int64),
        ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("n_splits", ctypes.c_int32),
        ("n_items", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64),
        ("launch_xcds", ctypes.c_int32), ("launch_per_xcd", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32), ("n_qblocks", ctypes.c_int32),
        ("n_kvblocks", ctypes.c_int32), ("n_tiles", ctypes.c_int32), ("computed_pairs_per_head", ctypes.c_int64),
    ]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libwa.so`` (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m chunk_windowed_softmax_amd.build`")
    # torch brings its own HIP runtime; load it first so that libwa.so binds to the same
    # runtime instance as the tensors and streams it is handed.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.wa_plan_create.argtypes = [ctypes.c_int] * 7 + [ctypes.POINTER(P)]
    lib.wa_causal_plan_create.argtypes = [ctypes.c_int] * 3 + [ctypes.POINTER(P)]
    lib.wa_blocksparse_plan_create.argtypes = [ctypes.c_int] * 9 + [ctypes.POINTER(P)]
    lib.wa_plan_block_mask.argtypes = [P, i32p, i32p, i32p, i32p, ctypes.c_size_t]
    lib.wa_plan_tiles.argtypes = [P, i32p, ctypes.c_size_t]
    lib.wa_plan_release.argtypes = [P]
    lib.wa_forward.argtypes = [P, P, P, P, P, ctypes.c_int, P]
    lib.wa_plan_info.argtypes = [P, ctypes.POINTER(_PlanInfo)]
    lib.wa_plan_groups.argtypes = [P, i32p, ctypes.c_size_t]
    lib.wa_plan_kv_indices.argtypes = [P, ctypes.c_int, i32p, ctypes.c_size_t]
    lib.wa_plan_items.argtypes = [P, i32p, ctypes.c_size_t]
    lib.wa_plan_launch_order.argtypes = [P, i32p, ctypes.c_size_t]
    lib.wa_forward_fp8.argtypes = [P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float, P, P]
    lib.wa_forward_noalloc.argtypes = [P, P, P, P, P, ctypes.c_int, P]
    lib.wa_qk_norm_rope.argtypes = [P] * 8 + [ctypes.c_int] * 3 + [ctypes.c_float] + [ctypes.c_int] * 2 + [P]
    lib.wa_last_error.argtypes = []
    lib.wa_last_error.restype = ctypes.c_char_p
    for name in EXPORTED_SYMBOLS:
        if name != "wa_last_error":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def wa_last_error() -> str:
    return load_library().wa_last_error().decode()


def _check(code: int) -> None:
    if code != WA_OK:
        raise WaError(code, wa_last_error())


class Plan:
    """Handle of a cached plan (one reference, released on garbage collection)."""

    def __init__(self, handle: ctypes.c_void_p):
        self._h = handle
        self.info = wa_plan_info(self)

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def release(self) -> None:
        if self._h:
            _check(load_library().wa_plan_release(self._h))
            self._h = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


def wa_plan_create(T: int, S: int, G: int, K: int, radius: int, H: int, d: int) -> Plan:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.wa_plan_create(T, S, G, K, radius, H, d, ctypes.byref(h)))
    return Plan(h)


def wa_causal_plan_create(n: int, H: int, d: int) -> Plan:
    """Plan for causal dense attention over n rows ([n, H, d] tensors; row i sees keys 0..i)."""
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.wa_causal_plan_create(n, H, d, ctypes.byref(h)))
    return Plan(h)


def wa_blocksparse_plan_create(T: int, S: int, G: int, K: int, radius: int, H: int, d: int, block_q: int,
                               block_kv: int) -> Plan:
    """Block-sparse plan of the window attention (block mask at (block_q, block_kv))."""
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.wa_blocksparse_plan_create(T, S, G, K, radius, H, d, block_q, block_kv, ctypes.byref(h)))
    return Plan(h)


def wa_plan_block_mask(plan: Plan):
    """(kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices) of a block-sparse plan:
    [n_qblocks], [n_qblocks, n_kvblocks] (unused entries -1), [n_qblocks], [n_qblocks, n_kvblocks]."""
    nq, nk = plan.info["n_qblocks"], plan.info["n_kvblocks"]
    kn, knp = _int32_buffer(nq)
    fn, fnp = _int32_buffer(nq)
    ki, kip = _int32_buffer(nq * nk)
    fi, fip = _int32_buffer(nq * nk)
    _check(load_library().wa_plan_block_mask(plan.handle, knp, kip, fnp, fip, nq * nk))
    return kn[:nq], ki[:nq * nk].reshape(nq, nk), fn[:nq], fi[:nq * nk].reshape(nq, nk)


def wa_plan_tiles(plan: Plan) -> np.ndarray:
    """Tile-list entries of a block-sparse plan's items: (first key row << 1) | needs_mask."""
    n = plan.info["n_tiles"]
    arr, ptr = _int32_buffer(n)
    _check(load_library().wa_plan_tiles(plan.handle, ptr, arr.size))
    return arr[:n]


def wa_plan_info(plan: Plan) -> dict:
    info = _PlanInfo()
    _check(load_library().wa_plan_info(plan.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in _PlanInfo._fields_}


def _int32_buffer(n: int):
    arr = np.zeros(max(n, 1), dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def wa_plan_groups(plan: Plan) -> np.ndarray:
    n = plan.info["n_groups"] * 6
    arr, ptr = _int32_buffer(n)
    _check(load_library().wa_plan_groups(plan.handle, ptr, arr.size))
    return arr[:n].reshape(-1, 6)


def wa_plan_kv_indices(plan: Plan, g: int) -> np.ndarray:
    groups = wa_plan_groups(plan)
    if not 0 <= g < len(groups):
        n = 1
    else:
        n = int(groups[g, 3] - groups[g, 2]) + plan.info["G"]
    arr, ptr = _int32_buffer(n)
    _check(load_library().wa_plan_kv_indices(plan.handle, g, ptr, arr.size))
    return arr[:n]


def wa_plan_items(plan: Plan) -> np.ndarray:
    n = plan.info["n_items"] * WA_ITEM_COLS
    arr, ptr = _int32_buffer(n)
    _check(load_library().wa_plan_items(plan.handle, ptr, arr.size))
    return arr[:n].reshape(-1, WA_ITEM_COLS)


def wa_plan_launch_order(plan: Plan) -> np.ndarray:
    """[launch_xcds, launch_per_xcd] int32: the work unit (head * n_items + item) of each
    block's slot, -1 for none."""
    x, per = plan.info["launch_xcds"], plan.info["launch_per_xcd"]
    arr, ptr = _int32_buffer(x * per)
    _check(load_library().wa_plan_launch_order(plan.handle, ptr, arr.size))
    return arr[: x * per].reshape(x, per)


def wa_forward(plan: Plan, q, k, v, out=None, stream=None):
    """Run the decomposed window attention; returns ``out`` ([L, H, d], dtype of q).

    q, k, v: contiguous CUDA (HIP) tensors [L, H, d] of one dtype, bfloat16 or float32.
    ``stream``: a torch stream (default: the current stream).
    """
    return _forward("wa_forward", plan, q, k, v, out, stream)


def wa_forward_noalloc(plan: Plan, q, k, v, out, stream=None):
    """wa_forward through the entry point that allocates nothing (its partial results and
    tables live in the library's static per-GPU workspace); ``out`` must be given."""
    if out is None:
        raise ValueError("wa_forward_noalloc needs a preallocated out")
    return _forward("wa_forward_noalloc", plan, q, k, v, out, stream)


def prepared_forward(plan: Plan, q, k, v, out, stream=None, noalloc: bool = False):
    """Check the arguments of ``wa_forward`` (or ``wa_forward_noalloc``) once and return a
    callable that repeats the call on the same tensors and stream with no further Python
    work than the C call (raises on a non-zero status)."""
    import torch

    _forward("wa_forward_noalloc" if noalloc else "wa_forward", plan, q, k, v, out, stream)  # validates, runs once
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = getattr(load_library(), "wa_forward_noalloc" if noalloc else "wa_forward")
    args = (plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            WA_F32 if q.dtype == torch.float32 else WA_BF16, ctypes.c_void_p(stream.cuda_stream))

    def call():
        _check(fn(*args))

    return call


def _forward(entry: str, plan: Plan, q, k, v, out, stream):
    import torch

    info = plan.info
    shape = (info["L"], info["H"], info["d"])
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {dtype}; use bfloat16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {shape}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=q.device)
    elif tuple(out.shape) != shape or out.dtype != dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous GPU tensor with the shape and dtype of q")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    code = WA_F32 if dtype == torch.float32 else WA_BF16
    with torch.cuda.device(q.device):
        _check(getattr(load_library(), entry)(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                              code, ctypes.c_void_p(stream.cuda_stream)))
    return out


def wa_forward_fp8(plan: Plan, q, k, v, scale_q: float, scale_k: float, scale_v: float, out=None, stream=None):
    """FP8 window attention; returns ``out`` ([L, H, d] bfloat16).

    q, k, v: contiguous GPU tensors [L, H, 128] of e4m3 codes (torch.float8_e4m3fn or
    uint8); the scales are their per-tensor dequantisation factors.
    """
    import torch

    info = plan.info
    shape = (info["L"], info["H"], info["d"])
    for name, t in (("q", q), ("k", k), ("v", v)):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {shape}")
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise ValueError(f"{name} must hold e4m3 codes (float8_e4m3fn or uint8), got {t.dtype}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
    elif tuple(out.shape) != shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous bfloat16 GPU tensor of the plan's shape")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        _check(load_library().wa_forward_fp8(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), scale_q, scale_k,
                                             scale_v, out.data_ptr(), ctypes.c_void_p(stream.cuda_stream)))
    return out


def wa_qk_norm_rope(q, k, cos, sin, wq=None, wk=None, eps: float = 1e-6, interleaved: bool = False,
                    q_out=None, k_out=None, stream=None):
    """RMSNorm of q and k, then the rotary embedding, in one launch; returns (q_out, k_out).

    q, k: contiguous GPU tensors [L, H, d] (bfloat16 or float32, d = 64 or 128).
    cos, sin: contiguous float32 GPU tensors [L, d/2].  wq, wk: float32 [d] or None.
    q_out / k_out default to new tensors; passing q / k itself works in place.
    """
    import torch

    if q.dim() != 3:
        raise ValueError("q must be [L, H, d]")
    L, H, d = q.shape
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {dtype}; use bfloat16 or float32")
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    for name, t in (("k", k), ("q_out", q_out), ("k_out", k_out)):
        if tuple(t.shape) != (L, H, d) or t.dtype != dtype:
            raise ValueError(f"{name} must have the shape and dtype of q")
    for name, t in (("cos", cos), ("sin", sin)):
        if tuple(t.shape) != (L, d // 2) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [L, d/2]")
    for name, t in (("wq", wq), ("wk", wk)):
        if t is not None and (tuple(t.shape) != (d,) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [d] or None")
    tensors = [t for t in (q, k, q_out, k_out, cos, sin, wq, wk) if t is not None]
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("every tensor must be a contiguous GPU tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(q.device):
        _check(load_library().wa_qk_norm_rope(
            ptr(q), ptr(k), ptr(q_out), ptr(k_out), ptr(cos), ptr(sin), ptr(wq), ptr(wk), L, H, d, eps,
            WA_ROPE_INTERLEAVED if interleaved else 0, WA_F32 if dtype == torch.float32 else WA_BF16,
            ctypes.c_void_p(stream.cuda_stream)))
    return q_out, k_out


__all__ = [
    "EXPORTED_SYMBOLS", "LIB_PATH", "Plan", "WaError", "WA_BF16", "WA_F32", "load_library", "wa_forward",
    "wa_last_error", "wa_plan_create", "wa_plan_groups", "wa_plan_info", "wa_plan_items", "wa_plan_kv_indices",
    "wa_plan_launch_order", "wa_causal_plan_create", "wa_qk_norm_rope", "WA_ROPE_INTERLEAVED", "wa_forward_fp8",
    "wa_forward_noalloc", "wa_blocksparse_plan_create", "wa_plan_block_mask", "wa_plan_tiles", "prepared_forward",
]
