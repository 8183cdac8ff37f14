"""Plain fp64 CPU oracle for chunk-windowed softmax attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU path never
imports it and shares no code with it; the two meet only through the seeded input
generators, which hold none of the method's arithmetic.

Sources (web pages; cited by title and section):

* [VDN] lqnn.cn article "VDN-Minimax-H3 window attention" -- the authority on the
  method.  §一 defines the packed sequence, HybridAttention's softmax window branch,
  the chunk-aligned window (``window_bounds``) and the fully connected global tokens.
  §三 states the decomposition (query rows with an identical kept-KV set form one
  dense attention), that the two legs' row sets are disjoint and cover the sequence,
  that the result equals the masked form exactly up to reduction order, and that a
  per-frame eager loop (``window_softmax_reference``) is kept as the correctness
  baseline.
* [VAE] prhub digest of sglang PR #34949 "H3 VAE attention via the native USP
  backend" -- the ``[B, L, H, d]`` q/k/v layout (``qkv.view(B, L, H, 3*d)``), the
  non-causal dense decoder, and SDPA called with its default 1/sqrt(d) scale.

Readings taken where the pages are silent:

* Row order: frames first, frame-major (row = t*S + s), then the G global rows.
* Windows are clipped to chunks [0, C-1]; the last chunk may hold fewer than K frames.
* Frame queries see every global key; global queries see every key (non-causal).
* Softmax scale 1/sqrt(d); inputs are not pre-scaled.
* Plan: only frame rows are grouped (maximal runs of chunks with identical windows);
  the global rows form the second leg with kv = [0, L).

Everything here is float64 computed from the exact input values (bf16 / fp32 inputs
are upcast exactly).  Every function is pinned by ``tests/test_oracle.py``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- geometry


@dataclass(frozen=True)
class Geometry:
    """Packed-sequence geometry ([VDN] §一).

    T latent frames of S spatial tokens each, then G global (text/audio) tokens.
    Chunks are K consecutive latent frames; ``radius`` is the chunk radius of the
    window.
    """

    T: int
    S: int
    G: int
    K: int
    radius: int

    @property
    def n_frame_rows(self) -> int:
        return self.T * self.S

    @property
    def L(self) -> int:
        return self.T * self.S + self.G

    @property
    def n_chunks(self) -> int:
        return -(-self.T // self.K)


def window_bounds(geom: Geometry, t: int) -> Tuple[int, int]:
    """Chunk window of latent frame ``t`` ([VDN] §一, ``window_bounds``).

    Frame t lies in chunk c = t // K and sees the whole chunks with index in
    [c - radius, c + radius]; the range is clipped to the chunks that exist.
    Returns (lo, hi), inclusive chunk indices.
    """
    c = t // geom.K
    return max(0, c - geom.radius), min(geom.n_chunks - 1, c + geom.radius)


def chunk_span_rows(geom: Geometry, lo: int, hi: int) -> Tuple[int, int]:
    """Row range [begin, end) covered by the whole chunks lo..hi (inclusive).

    The last chunk may be partial (T not a multiple of K), so the end is clipped
    to frame T.
    """
    return lo * geom.K * geom.S, min(geom.T, (hi + 1) * geom.K) * geom.S


def kept_set(geom: Geometry, i: int) -> np.ndarray:
    """Ascending kept-KV index set of query row ``i`` ([VDN] §一).

    A frame row keeps its window's chunk span plus every global row; a global row
    keeps the whole sequence.
    """
    if i >= geom.n_frame_rows:
        return np.arange(geom.L, dtype=np.int64)
    lo, hi = window_bounds(geom, i // geom.S)
    a, b = chunk_span_rows(geom, lo, hi)
    return np.concatenate([np.arange(a, b), np.arange(geom.n_frame_rows, geom.L)]).astype(np.int64)


def kept_pairs_per_head(geom: Geometry) -> int:
    """Number of kept (q, kv) pairs for one head, summed over all query rows."""
    total = 0
    for t in range(geom.T):
        lo, hi = window_bounds(geom, t)
        a, b = chunk_span_rows(geom, lo, hi)
        total += geom.S * ((b - a) + geom.G)
    total += geom.G * geom.L
    return total


# ----------------------------------------------------------------------------- plan


@dataclass(frozen=True)
class PlanGroup:
    q_begin: int
    q_end: int
    kv_begin: int
    kv_end: int
    chunk_lo: int
    chunk_hi: int


def plan_groups(geom: Geometry) -> List[PlanGroup]:
    """Window groups of the decomposed form ([VDN] §三).

    Query rows whose kept-KV sets are identical form one group.  For frame rows the
    kept set depends only on the window (lo, hi) of the row's chunk, so a group is a
    maximal run of consecutive chunks with the same window; its query rows are the
    rows of those chunks and its KV rows are the window's chunk span (followed by the
    global rows, which every frame row keeps).
    """
    groups: List[PlanGroup] = []
    C = geom.n_chunks
    c = 0
    while c < C:
        lo, hi = window_bounds(geom, c * geom.K)
        c_end = c
        while c_end + 1 < C and window_bounds(geom, (c_end + 1) * geom.K) == (lo, hi):
            c_end += 1
        q_begin, q_end = chunk_span_rows(geom, c, c_end)
        kv_begin, kv_end = chunk_span_rows(geom, lo, hi)
        groups.append(PlanGroup(q_begin, q_end, kv_begin, kv_end, lo, hi))
        c = c_end + 1
    return groups


def plan_kv_indices(geom: Geometry, g: PlanGroup) -> np.ndarray:
    """Explicit ascending kept-KV index list of a window group: span, then globals."""
    return np.concatenate(
        [np.arange(g.kv_begin, g.kv_end), np.arange(geom.n_frame_rows, geom.L)]
    ).astype(np.int64)


# ----------------------------------------------------------------------------- values


def _softmax_rows_fp64(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=-1, keepdims=True)


def _as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16 / fp16 / fp32 / fp64) or array to float64."""
    try:
        import torch  # local import: the oracle itself is numpy-only

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def window_attention_reference(q, k, v, geom: Geometry) -> np.ndarray:
    """Per-frame eager loop ([VDN] §三, ``window_softmax_reference``), in fp64.

    q, k, v: [L, H, d].  For every head and every latent frame t, the frame's S query
    rows attend to the kept set of t (its window's chunk span plus the global rows);
    then the G global rows attend to all L rows, in blocks of at most 128 rows.
    Scale 1/sqrt(d).  Returns float64 [L, H, d].
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    L, H, d = q.shape
    assert L == geom.L, (L, geom.L)
    scale = 1.0 / math.sqrt(d)
    out = np.empty((L, H, d), dtype=np.float64)
    glob = np.arange(geom.n_frame_rows, L)
    for h in range(H):
        for t in range(geom.T):
            rows = slice(t * geom.S, (t + 1) * geom.S)
            lo, hi = window_bounds(geom, t)
            a, b = chunk_span_rows(geom, lo, hi)
            keep = np.concatenate([np.arange(a, b), glob])
            p = _softmax_rows_fp64(scale * (q[rows, h] @ k[keep, h].T))
            out[rows, h] = p @ v[keep, h]
        for r0 in range(geom.n_frame_rows, L, 128):
            rows = slice(r0, min(L, r0 + 128))
            p = _softmax_rows_fp64(scale * (q[rows, h] @ k[:, h].T))
            out[rows, h] = p @ v[:, h]
    return out


def window_attention_rows(q, k, v, geom: Geometry, rows: Sequence[int], heads: Sequence[int]) -> np.ndarray:
    """Oracle output of selected query rows and heads only, one row at a time.

    Used to check outputs sampled from full-size runs.  Returns float64
    [len(rows), len(heads), d].
    """
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d)
    res = np.empty((len(rows), len(heads), d), dtype=np.float64)
    for a, i in enumerate(rows):
        keep = kept_set(geom, int(i))
        for b, h in enumerate(heads):
            qi = _as_f64(q[int(i), int(h)])
            kk = _as_f64(k[keep, int(h)])
            vv = _as_f64(v[keep, int(h)])
            s = scale * (kk @ qi)
            p = np.exp(s - s.max())
            res[a, b] = (p @ vv) / p.sum()
    return res


def window_mask(geom: Geometry) -> np.ndarray:
    """Explicit boolean [L, L] mask of the window rule, built pairwise ([VDN] §一).

    Frame rows i, j (frames t_i, t_j) are connected iff their chunks are at most
    ``radius`` apart; a pair involving a global row is always connected.
    """
    L, n = geom.L, geom.n_frame_rows
    chunk = np.full(L, -1, dtype=np.int64)
    chunk[:n] = (np.arange(n) // geom.S) // geom.K
    is_glob = np.arange(L) >= n
    close = np.abs(chunk[:, None] - chunk[None, :]) <= geom.radius
    return close | is_glob[:, None] | is_glob[None, :]


def masked_dense_attention(q, k, v, mask: np.ndarray) -> np.ndarray:
    """Brute-force dense attention with an explicit mask (disallowed pairs get -inf)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    L, H, d = q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    for h in range(H):
        s = scale * (q[:, h] @ k[:, h].T)
        s = np.where(mask, s, -np.inf)
        out[:, h] = _softmax_rows_fp64(s) @ v[:, h]
    return out
