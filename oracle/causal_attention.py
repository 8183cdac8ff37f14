"""Plain fp64 CPU oracle for causal dense attention (the audio-VAE attention).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU path never imports
it and shares no code with it.

Source (web page; cited by title and section):

* [VAE] prhub digest of sglang PR #34949 "H3 VAE attention via the native USP backend",
  item 3 (audio VAE) and its ``CausalAttention`` listing: the audio VAE's attention is
  causal scaled-dot-product attention over q, k, v laid out as (B, N, heads, head_dim);
  its released default runs in FP32, and when a fused backend is chosen the q/k/v are
  cast to that backend's dtype for the attention only, the output being returned in the
  input dtype.

Readings taken where the page is silent:

* Causal means query row i sees key rows 0..i (queries and keys have the same length,
  so the usual top-left alignment); the scale is SDPA's default 1/sqrt(head_dim).
* The fused-backend contract is modelled as: fp32 inputs rounded to bf16 (RNE) for the
  attention, fp32 output.  The oracle computes in float64 from the exact input values,
  so that rounding is part of the error the parity tolerance covers (as for the window
  path's fp32 case).

Every function is pinned by ``tests/test_oracle_causal.py``.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU) torch tensor of any float dtype."""
    if hasattr(x, "detach"):
        x = x.detach()
        if hasattr(x, "is_cuda") and x.is_cuda:
            x = x.cpu()
        import torch

        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def causal_pairs_per_head(n: int) -> int:
    """Kept (query, key) pairs of one head: row i keeps i + 1 keys."""
    return n * (n + 1) // 2


def causal_mask(n: int) -> np.ndarray:
    """[n, n] boolean, True where key j is visible to query i (j <= i)."""
    return np.tril(np.ones((n, n), dtype=bool))


def causal_attention_rows(q, k, v, rows: Sequence[int], heads: Sequence[int]) -> np.ndarray:
    """Output rows ``rows`` of heads ``heads``: [len(rows), len(heads), d] float64.

    Row i: softmax_j(q_i . k_j / sqrt(d)) over j = 0..i, applied to v_0..v_i, with the
    row max subtracted before exponentiation.
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    d = q64.shape[2]
    scale = 1.0 / math.sqrt(d)
    out = np.empty((len(rows), len(heads), d), dtype=np.float64)
    for a, i in enumerate(rows):
        for b, h in enumerate(heads):
            s = (k64[: i + 1, h, :] @ q64[i, h, :]) * scale
            p = np.exp(s - s.max())
            out[a, b, :] = (p @ v64[: i + 1, h, :]) / p.sum()
    return out


def causal_attention_reference(q, k, v, block: int = 256) -> np.ndarray:
    """All rows and heads: [n, H, d] float64.

    Query rows are taken in blocks; a block's rows see keys up to their own index, so
    each block computes scores against keys 0..(last row of the block) and masks the
    keys beyond each row's own index (set to -inf before the softmax).
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    n, H, d = q64.shape
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q64)
    for h in range(H):
        for r0 in range(0, n, block):
            r1 = min(n, r0 + block)
            s = (q64[r0:r1, h, :] @ k64[:r1, h, :].T) * scale  # [rows, keys 0..r1)
            rows = np.arange(r0, r1)[:, None]
            keys = np.arange(r1)[None, :]
            s = np.where(keys <= rows, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[r0:r1, h, :] = (p @ v64[:r1, h, :]) / p.sum(axis=1, keepdims=True)
    return out
