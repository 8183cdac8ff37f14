"""Named workloads and their seeded synthetic inputs.

This module holds geometry and random-number recipes only -- none of the attention
arithmetic -- so that both the HIP path's tests/benchmarks and the CPU oracle can be fed
the very same tensors.

Geometry comes from the VDN-Minimax-H3 window-attention article (lqnn.cn), §一: a
packed sequence of T latent frames x S spatial tokens followed by G global (text /
audio) tokens; chunks of K frames; window radius in chunks.  The head count and
head size of the H3-scale workload follow sglang PR #43164 (56 heads, 7 per GPU under
8-way head parallelism, head size 128).  The dense degenerate case is the non-causal
video-VAE ViT decoder of sglang PR #34949.

Input recipe (all configs): ``g = torch.Generator('cpu').manual_seed(seed)``; q, k, v
are drawn with ``torch.randn(L, H, d, generator=g)`` in that order (fp32), then cast
to the workload dtype with round-to-nearest-even.  For the ragged workload, a further
``torch.randperm(L, generator=g)[:round(0.01 * L)]`` picks rows whose q and k are
multiplied by 8 (exact in bf16) to stretch the softmax range.

The ``audio_causal*`` workloads are the causal dense attention of the audio VAE (the
prhub digest of sglang PR #34949, item 3): one sequence of L = S rows, row i attending to
rows 0..i, fp32 inputs and outputs.  The page states no sequence length or head shape;
16384 rows x 16 heads of 64 is a synthetic stand-in of long-clip scale.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    S: int
    G: int
    K: int
    radius: int
    H: int
    d: int
    dtype: torch.dtype
    scaled_row_frac: float = 0.0
    description: str = ""
    causal: bool = False  # causal dense attention over L = S rows (T = 1, G = 0)

    @property
    def L(self) -> int:
        return self.T * self.S + self.G

    @property
    def geometry(self) -> Tuple[int, int, int, int, int]:
        return (self.T, self.S, self.G, self.K, self.radius)

    def with_heads(self, H: int) -> "Workload":
        return Workload(self.name + f"_H{H}", self.T, self.S, self.G, self.K, self.radius, H, self.d,
                        self.dtype, self.scaled_row_frac, self.description, self.causal)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", T=6, S=16, G=8, K=2, radius=1, H=1, d=64, dtype=torch.float32,
                     description="6 frames x 16 tokens, K=2, radius 1, 8 globals, fp32"),
    "small": Workload("small", T=24, S=256, G=256, K=3, radius=1, H=8, d=128, dtype=torch.bfloat16,
                      description="24 frames x 256 tokens, K=3, radius 1, 256 globals, bf16"),
    "h3": Workload("h3", T=102, S=960, G=1024, K=3, radius=1, H=7, d=128, dtype=torch.bfloat16,
                   description="H3-scale one-GPU share: 102 latent frames x 960 tokens, K=3, radius 1, "
                               "1024 globals, 7 heads (56/8), bf16"),
    "h3_full": Workload("h3_full", T=102, S=960, G=1024, K=3, radius=1, H=56, d=128, dtype=torch.bfloat16,
                        description="H3 scale with all 56 heads, bf16"),
    "ragged": Workload("ragged", T=50, S=432, G=77, K=4, radius=2, H=16, d=128, dtype=torch.bfloat16,
                       scaled_row_frac=0.01,
                       description="50 frames (last chunk partial) x 432 tokens, K=4, radius 2, 77 globals, "
                                   "1% of rows with q,k scaled x8, bf16"),
    "dense": Workload("dense", T=8, S=1024, G=0, K=1, radius=8, H=16, d=64, dtype=torch.bfloat16,
                      description="degenerate dense ViT case: radius >= chunk count, no globals, bf16"),
    # Causal dense attention of the audio VAE (sglang PR #34949, item 3): fp32 in and out.
    # The page gives no sequence length or head shape; these are synthetic stand-ins.
    "audio_causal_small": Workload("audio_causal_small", T=1, S=1000, G=0, K=1, radius=0, H=2, d=64,
                                   dtype=torch.float32, causal=True,
                                   description="causal, 1000 rows, 2 heads of 64, fp32"),
    "audio_causal": Workload("audio_causal", T=1, S=16384, G=0, K=1, radius=0, H=16, d=64,
                             dtype=torch.float32, causal=True,
                             description="causal, 16384 rows, 16 heads of 64, fp32 in/out"),
}


def make_inputs(w: Workload, seed: int = 0, device: str = "cpu"):
    """Seeded q, k, v of shape [L, H, d] in the workload dtype (see module docstring)."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (w.L, w.H, w.d)
    q = torch.randn(shape, generator=g)
    k = torch.randn(shape, generator=g)
    v = torch.randn(shape, generator=g)
    if w.scaled_row_frac > 0:
        n = int(round(w.scaled_row_frac * w.L))
        idx = torch.randperm(w.L, generator=g)[:n]
        q[idx] *= 8.0
        k[idx] *= 8.0
    q, k, v = (x.to(w.dtype) for x in (q, k, v))
    if device != "cpu":
        q, k, v = (x.to(device) for x in (q, k, v))
    return q, k, v


def make_custom_inputs(L: int, H: int, d: int, dtype: torch.dtype, seed: int = 0, device: str = "cpu"):
    """Seeded q, k, v for an arbitrary geometry (same recipe, no scaled rows)."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((L, H, d), generator=g)
    k = torch.randn((L, H, d), generator=g)
    v = torch.randn((L, H, d), generator=g)
    q, k, v = (x.to(dtype) for x in (q, k, v))
    if device != "cpu":
        q, k, v = (x.to(device) for x in (q, k, v))
    return q, k, v


def make_rope_tables(L: int, d: int, base: float = 10000.0, device: str = "cpu"):
    """Angle tables cos, sin [L, d/2] (fp32) for the QK-norm + rotary prologue: row t's
    angle for channel pair j is t * base^(-2j/d), the common one-dimensional frequency
    ladder, with the row index as position (a synthetic stand-in: the pages give no
    positions or frequencies)."""
    pos = torch.arange(L, dtype=torch.float64)[:, None]
    freq = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = pos * freq[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    if device != "cpu":
        cos, sin = cos.to(device), sin.to(device)
    return cos, sin


def make_norm_weights(d: int, seed: int = 0, device: str = "cpu"):
    """Per-channel RMSNorm weights (wq, wk) [d] fp32: 1 + 0.1 * randn (seeded)."""
    g = torch.Generator("cpu").manual_seed(seed + 1000)
    wq = 1.0 + 0.1 * torch.randn(d, generator=g)
    wk = 1.0 + 0.1 * torch.randn(d, generator=g)
    if device != "cpu":
        wq, wk = wq.to(device), wk.to(device)
    return wq, wk


def make_prologue_inputs(L: int, H: int, d: int, dtype=torch.bfloat16, seed: int = 0, device: str = "cpu"):
    """q, k [L, H, d] for the QK-norm + rotary prologue: standard normal channels, each
    (row, head) vector scaled by 10^u with u uniform in [-2, 2] so the norm sees a spread
    of magnitudes (projection outputs before the norm are not unit-scaled)."""
    g = torch.Generator("cpu").manual_seed(seed)
    out = []
    for _ in range(2):
        x = torch.randn(L, H, d, generator=g)
        x *= 10.0 ** (4.0 * torch.rand(L, H, 1, generator=g) - 2.0)
        out.append(x.to(dtype).to(device) if device != "cpu" else x.to(dtype))
    return out[0], out[1]


def quantize_e4m3(x: torch.Tensor):
    """(codes, scale): per-tensor e4m3 quantisation of a float tensor, scale = amax / 448 (the
    largest e4m3 magnitude), codes = x / scale rounded to e4m3 by torch, as uint8."""
    scale = float(x.abs().max()) / 448.0
    if scale == 0.0:
        scale = 1.0
    codes = (x.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_fp8_inputs(w: Workload, seed: int = 0, device: str = "cpu"):
    """e4m3 codes of the workload's q, k, v (the make_inputs recipe in fp32) and their
    per-tensor scales: (q8, k8, v8, scale_q, scale_k, scale_v)."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (w.L, w.H, w.d)
    xs = [torch.randn(shape, generator=g) for _ in range(3)]
    if w.scaled_row_frac > 0:
        n = int(round(w.scaled_row_frac * w.L))
        idx = torch.randperm(w.L, generator=g)[:n]
        xs[0][idx] *= 8.0
        xs[1][idx] *= 8.0
    out = [quantize_e4m3(x) for x in xs]
    codes = [c if device == "cpu" else c.to(device) for c, _ in out]
    return codes[0], codes[1], codes[2], out[0][1], out[1][1], out[2][1]
