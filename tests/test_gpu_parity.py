"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (bf16 products, fp32 softmax and accumulation, output rounded to the input
dtype): relative L2 error <= 5e-3 and max abs error <= 2e-2 against the oracle evaluated
on the exact input values.  fp32 inputs are rounded to bf16 for the products, under the
same bound.
"""

import sys

import numpy as np
import pytest
import torch

from chunk_windowed_softmax_amd.workloads import WORKLOADS, make_custom_inputs, make_inputs
from oracle import (Geometry, causal_attention_reference, causal_attention_rows, window_attention_reference,
                    window_attention_rows)

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
MAX_ABS = 2e-2


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.abs(got - ref).max()
    return rel, mx


def _run(wa, w, q, k, v, out=None):
    plan = wa.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, q.shape[1], q.shape[2])
    o = wa.wa_forward(plan, q, k, v, out=out)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name", ["tiny", "small", "dense"])
def test_full_parity(gpu_lib, name):
    w = WORKLOADS[name]
    _say(f"full parity {name}: T={w.T} S={w.S} G={w.G} K={w.K} r={w.radius} H={w.H} d={w.d} {w.dtype}")
    q, k, v = make_inputs(w, seed=0)
    ref = window_attention_reference(q, k, v, Geometry(*w.geometry))
    out = _run(gpu_lib, w, q.cuda(), k.cuda(), v.cuda())
    assert out.dtype == w.dtype and tuple(out.shape) == (w.L, w.H, w.d)
    rel, mx = _errors(out.float().cpu(), ref)
    _say(f"{name}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def test_ragged_parity(gpu_lib):
    w = WORKLOADS["ragged"]
    _say("ragged parity (heads 0, 7, 15 in full; all heads on sampled rows)")
    q, k, v = make_inputs(w, seed=0)
    out = _run(gpu_lib, w, q.cuda(), k.cuda(), v.cuda()).float().cpu()
    heads = [0, 7, 15]
    ref = window_attention_reference(q[:, heads], k[:, heads], v[:, heads], Geometry(*w.geometry))
    rel, mx = _errors(out[:, heads], ref)
    _say(f"ragged heads {heads}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(w.L, 48, replace=False), [0, w.T * w.S - 1, w.T * w.S, w.L - 1]]))
    ref_rows = window_attention_rows(q, k, v, Geometry(*w.geometry), rows, range(w.H))
    rel, mx = _errors(out[rows], ref_rows)
    _say(f"ragged sampled rows: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    n_frame = w.T * w.S
    edges = [0, w.S - 1, n_frame - 1, n_frame, w.L - 1]
    chunk_rows = w.K * w.S
    edges += [c * chunk_rows for c in range(1, 4)] + [c * chunk_rows - 1 for c in range(1, 4)]
    picks = rng.choice(w.L, n, replace=False)
    glob = n_frame + rng.choice(w.G, min(16, w.G), replace=False) if w.G else []
    return np.unique(np.concatenate([picks, edges, glob]).astype(np.int64))


@pytest.mark.parametrize("name", ["h3", "h3_full"])
def test_h3_scale_sampled_parity(gpu_lib, name):
    w = WORKLOADS[name]
    _say(f"{name}: generating inputs L={w.L} H={w.H}")
    q, k, v = make_inputs(w, seed=0)
    _say(f"{name}: running")
    out = _run(gpu_lib, w, q.cuda(), k.cuda(), v.cuda())
    assert not torch.isnan(out).any()
    out = out.cpu()
    rows = _sample_rows(w, 96 if w.H <= 8 else 24, seed=2)
    heads = list(range(w.H)) if w.H <= 8 else [0, 13, 27, 41, 55]
    _say(f"{name}: oracle on {len(rows)} rows x {len(heads)} heads")
    ref = window_attention_rows(q, k, v, Geometry(*w.geometry), rows, heads)
    rel, mx = _errors(out[rows][:, heads].float(), ref)
    _say(f"{name} sampled: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


@pytest.mark.parametrize("geom,H,d,dtype", [
    ((1, 1, 0, 1, 0), 1, 64, torch.bfloat16),      # one row
    ((3, 5, 1, 2, 0), 2, 128, torch.bfloat16),     # tiny ragged rows, one global
    ((13, 7, 3, 5, 1), 3, 64, torch.float32),      # last chunk partial, fp32
    ((9, 33, 130, 2, 3), 2, 128, torch.bfloat16),  # radius >= chunks with globals; 2 global tiles
    ((11, 70, 65, 3, 1), 1, 128, torch.bfloat16),  # rows not a multiple of 32/64/128
    ((40, 48, 200, 1, 2), 2, 64, torch.bfloat16),  # K = 1, many groups, split global leg
    ((6, 300, 40, 1, 1), 2, 128, torch.bfloat16),  # 44-row window and 40-row global items
    ((7, 60, 33, 1, 2), 3, 64, torch.float32),     # every item one wave (60-row chunks)
])
def test_edge_geometries(gpu_lib, geom, H, d, dtype):
    T, S, G, K, r = geom
    _say(f"edge geometry T={T} S={S} G={G} K={K} r={r} H={H} d={d} {dtype}")
    L = T * S + G
    q, k, v = make_custom_inputs(L, H, d, dtype, seed=3)
    plan = gpu_lib.wa_plan_create(T, S, G, K, r, H, d)
    out = gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    ref = window_attention_reference(q, k, v, Geometry(T, S, G, K, r))
    rel, mx = _errors(out.float().cpu(), ref)
    _say(f"rel_l2={rel:.3e} max_abs={mx:.3e} splits={plan.info['n_splits']}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def test_cover_determinism_locality(gpu_lib):
    """Every output element written (NaN prefill), bitwise repeatable, and keys outside a
    row's window are never read (perturbing them leaves those rows bit-identical)."""
    w = WORKLOADS["small"]
    _say("cover / determinism / locality on small")
    q, k, v = (x.cuda() for x in make_inputs(w, seed=4))
    plan = gpu_lib.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    out1 = torch.full_like(q, float("nan"))
    gpu_lib.wa_forward(plan, q, k, v, out=out1)
    out2 = torch.full_like(q, float("nan"))
    gpu_lib.wa_forward(plan, q, k, v, out=out2)
    torch.cuda.synchronize()
    assert not torch.isnan(out1).any()
    assert torch.equal(out1, out2)
    # chunk 0 (frames 0..2) sees chunks 0..1 = rows [0, 1536) plus globals
    span_end = 2 * w.K * w.S
    k2, v2 = k.clone(), v.clone()
    k2[span_end:w.T * w.S] = 7.0
    v2[span_end:w.T * w.S] = -7.0
    out3 = gpu_lib.wa_forward(plan, q, k2, v2)
    torch.cuda.synchronize()
    first_chunk = w.K * w.S
    assert torch.equal(out3[:first_chunk], out1[:first_chunk])
    assert not torch.equal(out3[first_chunk:2 * first_chunk], out1[first_chunk:2 * first_chunk])


def test_rows_sum_to_one_and_fp32_output(gpu_lib):
    w = WORKLOADS["tiny"]
    _say("ones-V on tiny (fp32)")
    q, k, _ = make_inputs(w, seed=5)
    v = torch.ones_like(q)
    out = _run(gpu_lib, w, q.cuda(), k.cuda(), v.cuda())
    assert out.dtype == torch.float32
    assert (out - 1).abs().max().item() <= 4e-3


def _hot_key(q, k, row, key, factor):
    """Make key `key` of every head the direction of q[row] scaled by `factor`, so that
    row `row` scores it about factor * |q|^2 / sqrt(d) (hundreds here): far above anything
    earlier in the row, beyond what exponentials against a stale running max can hold."""
    k[key] = (q[row].float() * factor).to(k.dtype)


def test_score_jump_parity(gpu_lib):
    """Scores that jump far above the running max after a unit's first tile, in window
    rows and in global rows (the split global leg): exponentials against the stale max
    would overflow, so the per-tile test must send those tiles to the slow path."""
    T, S, G, K, r, H, d = 4, 256, 64, 1, 3, 2, 128
    _say(f"score jump T={T} S={S} G={G} K={K} r={r} H={H} d={d}")
    L = T * S + G
    q, k, v = make_custom_inputs(L, H, d, torch.bfloat16, seed=9)
    _hot_key(q, k, 5, 900, 10.0)         # window row, key in a late tile of its unit
    _hot_key(q, k, T * S + 10, 700, 10.0)  # global row
    _hot_key(q, k, 300, 1030, 12.0)      # window row, hot key among the global keys
    plan = gpu_lib.wa_plan_create(T, S, G, K, r, H, d)
    out = gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    ref = window_attention_reference(q, k, v, Geometry(T, S, G, K, r))
    got = out.float().cpu()
    rel, mx = _errors(got, ref)
    _say(f"rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert not torch.isnan(got).any()
    assert rel <= REL_L2 and mx <= MAX_ABS
    # the hot rows are (almost) one-hot on their key
    for row, key in ((5, 900), (T * S + 10, 700), (300, 1030)):
        assert np.abs(got[row].numpy() - v[key].float().numpy()).max() <= 2e-2, row


def test_score_jump_causal(gpu_lib):
    # bf16 inputs: products of exactly representable values, so scores in the hundreds
    # carry no input-rounding error (fp32 inputs would be rounded to bf16 first, and an
    # error of a fraction of a unit in such scores moves the softmax weights visibly)
    n, H, d = 1000, 1, 64
    _say(f"score jump causal n={n} H={H} d={d}")
    q, k, v = make_custom_inputs(n, H, d, torch.bfloat16, seed=10)
    _hot_key(q, k, 900, 500, 12.0)  # key 500: a fast-path tile of row 900's item
    plan = gpu_lib.wa_causal_plan_create(n, H, d)
    out = gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    ref = causal_attention_reference(q, k, v)
    rel, mx = _errors(out.float().cpu(), ref)
    _say(f"causal score jump: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


# ---------------------------------------------------------------- causal (audio VAE)


@pytest.mark.parametrize("n,H,d,dtype", [
    (1, 1, 64, torch.float32),      # one row
    (37, 2, 64, torch.float32),     # inside one key tile
    (256, 2, 128, torch.bfloat16),  # exactly one work item
    (300, 3, 64, torch.float32),    # ragged second item
    (1000, 2, 64, torch.float32),   # several items, ragged tail
    (777, 1, 128, torch.bfloat16),
])
def test_causal_parity(gpu_lib, n, H, d, dtype):
    _say(f"causal parity n={n} H={H} d={d} {dtype}")
    q, k, v = make_custom_inputs(n, H, d, dtype, seed=6)
    plan = gpu_lib.wa_causal_plan_create(n, H, d)
    out = gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    assert out.dtype == dtype and tuple(out.shape) == (n, H, d)
    ref = causal_attention_reference(q, k, v)
    rel, mx = _errors(out.float().cpu(), ref)
    _say(f"causal n={n}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def test_audio_causal_sampled_parity(gpu_lib):
    w = WORKLOADS["audio_causal"]
    _say(f"audio_causal: L={w.L} H={w.H} d={w.d} fp32")
    q, k, v = make_inputs(w, seed=0)
    plan = gpu_lib.wa_causal_plan_create(w.L, w.H, w.d)
    out = gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    out = out.cpu()
    assert out.dtype == torch.float32 and not torch.isnan(out).any()
    rng = np.random.default_rng(7)
    edges = [0, 1, 31, 32, 63, 64, 65, 255, 256, 257, 4095, 4096, w.L - 2, w.L - 1]
    rows = np.unique(np.concatenate([rng.choice(w.L, 48, replace=False), edges]).astype(np.int64))
    _say(f"audio_causal: oracle on {len(rows)} rows x {w.H} heads")
    ref = causal_attention_rows(q, k, v, rows, range(w.H))
    rel, mx = _errors(out[rows].float(), ref)
    _say(f"audio_causal sampled: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def test_causal_cover_determinism_and_no_future_keys(gpu_lib):
    """NaN prefill is fully overwritten, results repeat bit for bit, and perturbing rows
    >= j of k and v leaves output rows < j bit-identical (future keys are never used)."""
    n, H, d = 700, 2, 64
    _say("causal cover / determinism / future keys")
    q, k, v = (x.cuda() for x in make_custom_inputs(n, H, d, torch.bfloat16, seed=8))
    plan = gpu_lib.wa_causal_plan_create(n, H, d)
    out1 = torch.full_like(q, float("nan"))
    gpu_lib.wa_forward(plan, q, k, v, out=out1)
    out2 = torch.full_like(q, float("nan"))
    gpu_lib.wa_forward(plan, q, k, v, out=out2)
    torch.cuda.synchronize()
    assert not torch.isnan(out1).any() and torch.equal(out1, out2)
    for j in (1, 100, 256, 321, 699):
        k2, v2 = k.clone(), v.clone()
        k2[j:] = 3.0
        v2[j:] = -5.0
        out3 = gpu_lib.wa_forward(plan, q, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(out3[:j], out1[:j]), j
        assert not torch.equal(out3[j:], out1[j:]), j
