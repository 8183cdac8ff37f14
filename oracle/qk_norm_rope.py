"""Plain fp64 CPU oracle for the QK-RMSNorm + rotary-embedding prologue of the attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU path never imports
it and shares no code with it.

Sources (web pages; cited by title and section):

* [VAE] prhub digest of sglang PR #34949 "H3 VAE attention via the native USP backend",
  the ViT ``Attention.forward`` listing: after the qkv projection is split into q, k, v of
  shape (batch, tokens, heads, head_dim), q and k go through ``qk_norm`` and the rotary
  position embedding (``rotary_pos_emb``, handed to ``forward``) before the attention; the
  digest's test list names a contract test for an affine-free RMSNorm as ``qk_norm``.
* [USP] sglang PR #43164 (MiniMax-H3 Ulysses exchange), Modifications item 2: one
  out-of-place kernel normalises q and k, applies RoPE and writes them (and v) to their
  destination, instead of an in-place norm followed by a copy.

Readings taken where the pages are silent:

* The norm is RMSNorm over each (token, head) vector of head_dim channels:
  ``y = x / sqrt(mean(x^2) + eps) * w``, with an optional per-channel weight ``w`` shared
  by all tokens and heads (separate for q and k) or none (the affine-free form); ``eps``
  is a parameter.
* The rotary embedding rotates channel pairs of the normalised vector by per-token
  angles, given as tables ``cos[t, j]``, ``sin[t, j]`` for j < head_dim / 2 (the caller
  computes the angles, as ``rotary_pos_emb`` is handed in).  Pairs are (j, j + d/2)
  ("rotate half") by default, or (2j, 2j + 1) ("interleaved"); both conventions are in use.
* v is not changed.

Every function is pinned by ``tests/test_oracle_qk_norm_rope.py``.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU) torch tensor of any float dtype."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach()
        if hasattr(x, "is_cuda") and x.is_cuda:
            x = x.cpu()
        import torch

        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, w=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w (w = 1 when None)."""
    x = _as_f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if w is not None:
        y = y * _as_f64(w)
    return y


def rope(y, cos, sin, interleaved: bool = False) -> np.ndarray:
    """Rotary embedding of y [L, H, d] with angle tables cos, sin [L, d/2].

    Pair j is (j, j + d/2), or (2j, 2j + 1) when interleaved; it is rotated by the angle
    of row t and column j:  (a, b) -> (a cos - b sin, b cos + a sin).
    """
    y = _as_f64(y)
    c = _as_f64(cos)[:, None, :]
    s = _as_f64(sin)[:, None, :]
    d = y.shape[-1]
    if interleaved:
        a, b = y[..., 0::2], y[..., 1::2]
    else:
        a, b = y[..., : d // 2], y[..., d // 2:]
    ra = a * c - b * s
    rb = b * c + a * s
    out = np.empty_like(y)
    if interleaved:
        out[..., 0::2], out[..., 1::2] = ra, rb
    else:
        out[..., : d // 2], out[..., d // 2:] = ra, rb
    return out


def qk_norm_rope_reference(q, k, cos, sin, wq=None, wk=None, eps: float = 1e-6,
                           interleaved: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(q', k'): RMSNorm of every (token, head) vector (weights wq / wk), then the rotary
    embedding with the token's angles.  q, k: [L, H, d]; cos, sin: [L, d/2]."""
    return (rope(rms_norm(q, wq, eps), cos, sin, interleaved),
            rope(rms_norm(k, wk, eps), cos, sin, interleaved))
