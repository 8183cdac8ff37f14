"""GPU parity of the fused QK-RMSNorm + rotary prologue (wa_qk_norm_rope) against the
fp64 oracle, element by element.

Tolerance: the kernel computes in fp32 and rounds once to the output dtype.  For bf16
output the rounding alone is up to 2^-8 of the value; the fp32 steps (a 128-term sum of
squares, the reciprocal square root, the rotation) add a relative error of a few 1e-6 and
an absolute one near 1e-6 where the rotation cancels (normalised values are O(1)).  So
each element must satisfy |got - ref| <= rel * |ref| + 1e-5 with rel = 2^-8 (bf16) or
1e-5 (fp32), the oracle evaluated on the exact input values.
"""

import sys

import numpy as np
import pytest
import torch

from chunk_windowed_softmax_amd.workloads import make_norm_weights, make_prologue_inputs, make_rope_tables
from oracle import qk_norm_rope_reference

pytestmark = pytest.mark.gpu

ABS = 1e-5
REL = {torch.bfloat16: 2.0 ** -8, torch.float32: 1e-5}


def _say(msg):
    print(f"[gpu-prologue] {msg}", flush=True)
    sys.stdout.flush()


def _check(got, ref, dtype, what):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = REL[dtype] * np.abs(ref) + ABS
    worst = float((err / bound).max()) if err.size else 0.0
    _say(f"{what}: max_abs={err.max() if err.size else 0:.3e} worst err/bound={worst:.3f}")
    assert np.isfinite(got).all(), what
    assert (err <= bound).all(), what


def _case(wa, L, H, d, dtype, interleaved, weights, seed=0, random_angles=False, eps=1e-6):
    q, k = make_prologue_inputs(L, H, d, dtype, seed)
    if random_angles:
        g = torch.Generator("cpu").manual_seed(seed + 7)
        ang = (torch.rand(L, d // 2, generator=g, dtype=torch.float64) * 2 - 1) * np.pi
        cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    else:
        cos, sin = make_rope_tables(L, d)
    wq, wk = make_norm_weights(d, seed) if weights else (None, None)
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    qd, kd = dev(q), dev(k)
    qo, ko = wa.wa_qk_norm_rope(qd, kd, dev(cos), dev(sin), dev(wq), dev(wk), eps=eps, interleaved=interleaved)
    torch.cuda.synchronize()
    rq, rk = qk_norm_rope_reference(q, k, cos, sin, wq, wk, eps=eps, interleaved=interleaved)
    tag = f"L={L} H={H} d={d} {dtype} interleaved={interleaved} weights={weights}"
    assert qo.dtype == dtype and ko.dtype == dtype
    _check(qo, rq, dtype, "q " + tag)
    _check(ko, rk, dtype, "k " + tag)
    # out of place: the inputs are untouched
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k)


@pytest.mark.parametrize("weights", [False, True])
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_prologue_parity(gpu_lib, d, dtype, interleaved, weights):
    # 333 rows x 3 heads x 2 tensors: several blocks and a ragged last block for both d
    _case(gpu_lib, 333, 3, d, dtype, interleaved, weights, random_angles=True)


@pytest.mark.parametrize("L,H", [(1, 1), (5, 7), (17, 1)])
def test_prologue_small_shapes(gpu_lib, L, H):
    _case(gpu_lib, L, H, 128, torch.bfloat16, False, True, seed=3)
    _case(gpu_lib, L, H, 64, torch.float32, True, False, seed=4)


def test_prologue_eps_zero_and_position_tables(gpu_lib):
    _case(gpu_lib, 200, 2, 128, torch.float32, False, True, eps=0.0)
    _case(gpu_lib, 200, 2, 64, torch.bfloat16, True, True, eps=1e-2)


def test_prologue_zero_vector(gpu_lib):
    """A zero (row, head) vector normalises to zero (eps > 0), its neighbours are unaffected."""
    q, k = make_prologue_inputs(9, 4, 128, torch.bfloat16, seed=5)
    q[3, 2].zero_()
    k[0, 0].zero_()
    cos, sin = make_rope_tables(9, 128)
    qo, ko = gpu_lib.wa_qk_norm_rope(q.cuda(), k.cuda(), cos.cuda(), sin.cuda())
    torch.cuda.synchronize()
    rq, rk = qk_norm_rope_reference(q, k, cos, sin)
    assert (qo[3, 2].float() == 0).all() and (ko[0, 0].float() == 0).all()
    _check(qo, rq, torch.bfloat16, "q zero vector")
    _check(ko, rk, torch.bfloat16, "k zero vector")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prologue_in_place(gpu_lib, dtype):
    L, H, d = 150, 5, 128
    q, k = make_prologue_inputs(L, H, d, dtype, seed=6)
    cos, sin = make_rope_tables(L, d)
    wq, wk = make_norm_weights(d, 6)
    qd, kd = q.cuda(), k.cuda()
    qo, ko = gpu_lib.wa_qk_norm_rope(qd, kd, cos.cuda(), sin.cuda(), wq.cuda(), wk.cuda(), q_out=qd, k_out=kd)
    torch.cuda.synchronize()
    assert qo.data_ptr() == qd.data_ptr() and ko.data_ptr() == kd.data_ptr()
    rq, rk = qk_norm_rope_reference(q, k, cos, sin, wq, wk)
    _check(qd, rq, dtype, "q in place")
    _check(kd, rk, dtype, "k in place")


def test_prologue_empty(gpu_lib):
    q = torch.empty(0, 3, 128, dtype=torch.bfloat16, device="cuda")
    cos = torch.empty(0, 64, dtype=torch.float32, device="cuda")
    qo, ko = gpu_lib.wa_qk_norm_rope(q, q.clone(), cos, cos.clone())
    torch.cuda.synchronize()
    assert qo.shape == (0, 3, 128) and ko.shape == (0, 3, 128)


def test_prologue_h3_sampled(gpu_lib):
    """The H3 window shape (102 frames x 960 tokens + 1024 global tokens, 7 heads, d = 128,
    bf16) in the launch the benchmark times; the oracle checks 3000 sampled rows (first,
    last and random), which span the grid-stride passes of the capped launch."""
    L, H, d = 102 * 960 + 1024, 7, 128
    _say(f"h3 prologue L={L} H={H} d={d}")
    q, k = make_prologue_inputs(L, H, d, torch.bfloat16, seed=11)
    cos, sin = make_rope_tables(L, d)
    wq, wk = make_norm_weights(d, 11)
    qo, ko = gpu_lib.wa_qk_norm_rope(q.cuda(), k.cuda(), cos.cuda(), sin.cuda(), wq.cuda(), wk.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, L - 2, L - 1], rng.integers(0, L, 2996)]))
    idx = torch.from_numpy(rows)
    rq, rk = qk_norm_rope_reference(q[idx], k[idx], cos[idx], sin[idx], wq, wk)
    _check(qo.cpu()[idx], rq, torch.bfloat16, "q h3 sampled")
    _check(ko.cpu()[idx], rk, torch.bfloat16, "k h3 sampled")
