"""FP8 (e4m3) inputs of the FP8 attention path, decoded in fp64 -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module.  The GPU path never imports it and shares no code with it.

Sources:
* lqnn.cn article on VDN-Minimax-H3 window attention, §四: its fastest H3 configurations are
  FP8 ones; it does not say which operands of the attention run in FP8.
* The OCP 8-bit floating point specification, E4M3 format: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; there are no
  infinities, and S.1111.111 is NaN (so the largest finite magnitude is 1.75 * 2^8 = 448).

Reading: an FP8 tensor is a tensor of e4m3 codes with one fp32 scale per tensor, value =
decoded code * scale.  The attention of FP8 inputs is the plain attention of those values,
so the oracle decodes and calls the fp64 window (or causal) attention oracle.  Rounding the
softmax weights to e4m3 inside a kernel is that kernel's approximation, not part of the
definition.

Pinned by ``tests/test_oracle_fp8.py``.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .causal_attention import causal_attention_reference, causal_attention_rows
from .window_attention import Geometry, window_attention_reference, window_attention_rows


def decode_e4m3(codes) -> np.ndarray:
    """Exact float64 values of e4m3 codes (uint8 array or tensor; NaN for S.1111.111)."""
    if hasattr(codes, "detach"):
        codes = codes.detach().cpu()
        import torch

        if codes.dtype != torch.uint8:
            codes = codes.view(torch.uint8)
        codes = codes.numpy()
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _values(codes, scale: float) -> np.ndarray:
    return decode_e4m3(codes) * float(scale)


def fp8_window_attention_reference(q8, k8, v8, scale_q: float, scale_k: float, scale_v: float,
                                   geom: Geometry) -> np.ndarray:
    """Window attention of the decoded, scaled inputs ([L, H, d] codes -> [L, H, d] fp64)."""
    return window_attention_reference(_values(q8, scale_q), _values(k8, scale_k), _values(v8, scale_v), geom)


def fp8_window_attention_rows(q8, k8, v8, scale_q: float, scale_k: float, scale_v: float, geom: Geometry,
                              rows: Sequence[int], heads: Sequence[int]) -> np.ndarray:
    """Selected rows and heads of fp8_window_attention_reference."""
    return window_attention_rows(_values(q8, scale_q), _values(k8, scale_k), _values(v8, scale_v), geom, rows, heads)


def fp8_causal_attention_reference(q8, k8, v8, scale_q: float, scale_k: float, scale_v: float) -> np.ndarray:
    """Causal attention of the decoded, scaled inputs."""
    return causal_attention_reference(_values(q8, scale_q), _values(k8, scale_k), _values(v8, scale_v))


def fp8_causal_attention_rows(q8, k8, v8, scale_q: float, scale_k: float, scale_v: float,
                              rows: Sequence[int], heads: Sequence[int]) -> np.ndarray:
    return causal_attention_rows(_values(q8, scale_q), _values(k8, scale_k), _values(v8, scale_v), rows, heads)
