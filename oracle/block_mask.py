"""Block mask of the chunk-windowed attention at (block_q, block_kv) granularity.

TEST INFRASTRUCTURE ONLY (see the package header): checks the block-sparse plan of the HIP
library, never used by it.

Source: [VDN] lqnn.cn article "VDN-Minimax-H3 window attention", §二 -- the FlexAttention
path builds a block-level mask from the window rule (``build_window_block_mask`` /
``create_block_mask``) and computes whole blocks, so window edges round up to block edges;
§四 measures that path against the decomposed one.  The layout follows FlexAttention's
BlockMask: per query block, the key blocks kept in part (``kv_num_blocks`` /
``kv_indices``, which need the mask applied element by element) and those kept in full
(``full_kv_num_blocks`` / ``full_kv_indices``), ascending.

Readings (the page gives the mask's purpose, not its construction):

* Only the frame rows' queries are blocked: query block i covers rows
  [i*block_q, min(T*S, (i+1)*block_q)); the global rows' queries see every key and run as a
  separate leg.  Key block j covers keys [j*block_kv, min(L, (j+1)*block_kv)).
* A key block is "full" for a query block when every pair of the query block's rows and
  block_kv keys is kept (a key block cut short by the end of the sequence is never full);
  "partial" when some pair is kept; absent otherwise.  Unused index entries are -1.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .window_attention import Geometry, chunk_span_rows, window_bounds, window_mask


def block_mask(geom: Geometry, block_q: int, block_kv: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices) of the frame rows.

    Kept pairs of (query block i, key block j) are counted frame by frame: the rows of one
    frame keep their window's chunk span and the global rows (``window_bounds``,
    ``chunk_span_rows``), so each frame adds rows x |kept keys in the block|.
    """
    TS, L = geom.n_frame_rows, geom.L
    nq = -(-TS // block_q)
    nk = -(-L // block_kv)
    k0 = np.arange(nk, dtype=np.int64) * block_kv
    k1 = np.minimum(L, k0 + block_kv)
    kv_num = np.zeros(nq, np.int32)
    full_num = np.zeros(nq, np.int32)
    kv_idx = np.full((nq, nk), -1, np.int32)
    full_idx = np.full((nq, nk), -1, np.int32)
    in_glob = np.maximum(0, np.minimum(L, k1) - np.maximum(TS, k0))
    for i in range(nq):
        r0, r1 = i * block_q, min(TS, (i + 1) * block_q)
        kept = np.zeros(nk, np.int64)
        r = r0
        while r < r1:
            t = r // geom.S
            r_end = min(r1, (t + 1) * geom.S)
            a, b = chunk_span_rows(geom, *window_bounds(geom, t))
            in_span = np.maximum(0, np.minimum(b, k1) - np.maximum(a, k0))
            kept += (r_end - r) * (in_span + in_glob)
            r = r_end
        full = (k1 - k0 == block_kv) & (kept == (r1 - r0) * block_kv)
        part = (kept > 0) & ~full
        f, p = np.nonzero(full)[0], np.nonzero(part)[0]
        full_num[i], kv_num[i] = len(f), len(p)
        full_idx[i, :len(f)] = f
        kv_idx[i, :len(p)] = p
    return kv_num, kv_idx, full_num, full_idx


def block_mask_brute_force(geom: Geometry, block_q: int, block_kv: int):
    """The same block mask from the explicit pairwise [L, L] mask (``window_mask``): small
    geometries only."""
    m = window_mask(geom)[: geom.n_frame_rows]
    TS, L = geom.n_frame_rows, geom.L
    nq, nk = -(-TS // block_q), -(-L // block_kv)
    kv_num = np.zeros(nq, np.int32)
    full_num = np.zeros(nq, np.int32)
    kv_idx = np.full((nq, nk), -1, np.int32)
    full_idx = np.full((nq, nk), -1, np.int32)
    for i in range(nq):
        for j in range(nk):
            blk = m[i * block_q:(i + 1) * block_q, j * block_kv:(j + 1) * block_kv]
            if not blk.any():
                continue
            if blk.shape[1] == block_kv and blk.all():
                full_idx[i, full_num[i]] = j
                full_num[i] += 1
            else:
                kv_idx[i, kv_num[i]] = j
                kv_num[i] += 1
    return kv_num, kv_idx, full_num, full_idx


def block_sparse_computed_pairs(geom: Geometry, block_q: int, block_kv: int) -> int:
    """(query, key) pairs of the frame rows that a block-sparse evaluation computes: every
    row of a query block times the keys of its listed (partial or full) key blocks."""
    kv_num, kv_idx, full_num, full_idx = block_mask(geom, block_q, block_kv)
    TS, L = geom.n_frame_rows, geom.L
    total = 0
    for i in range(len(kv_num)):
        rows = min(TS, (i + 1) * block_q) - i * block_q
        blocks = np.concatenate([kv_idx[i, :kv_num[i]], full_idx[i, :full_num[i]]]).astype(np.int64)
        keys = np.minimum(L, (blocks + 1) * block_kv) - blocks * block_kv
        total += rows * int(keys.sum())
    return total
