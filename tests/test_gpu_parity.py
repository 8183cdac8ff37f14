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

from _oracle_pool import by_heads
from _oracle_pool import workers as by_heads_workers
from chunk_windowed_softmax_amd.workloads import WORKLOADS, make_custom_inputs, make_inputs
from oracle import (Geometry, causal_attention_reference, chunk_span_rows, plan_groups,
                    window_attention_reference, window_attention_rows, window_bounds)

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


@pytest.mark.parametrize("name", ["tiny", "small", "dense", "ragged", "h3"])
def test_full_parity(gpu_lib, name):
    """Every row and head of the workload against the fp64 oracle (per-frame loop)."""
    w = WORKLOADS[name]
    _say(f"full parity {name}: T={w.T} S={w.S} G={w.G} K={w.K} r={w.radius} H={w.H} d={w.d} {w.dtype}")
    q, k, v = make_inputs(w, seed=0)
    out = _run(gpu_lib, w, q.cuda(), k.cuda(), v.cuda())
    assert out.dtype == w.dtype and tuple(out.shape) == (w.L, w.H, w.d)
    out = out.float().cpu()
    _say(f"{name}: oracle on all {w.L} rows x {w.H} heads ({by_heads_workers()} threads)")
    ref = by_heads(window_attention_reference, q, k, v, Geometry(*w.geometry))
    rel, mx = _errors(out, ref)
    _say(f"{name}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def _h3_rows(w, n_random, seed):
    """Rows of every window group's first and last 256-row item (first and last row of
    each), of every 256-row global tile (first and last row), and `n_random` more."""
    geom = Geometry(*w.geometry)
    rows = []
    for g in plan_groups(geom):
        last = g.q_begin + (g.q_end - 1 - g.q_begin) // 256 * 256
        rows += [g.q_begin, min(g.q_end, g.q_begin + 256) - 1, last, g.q_end - 1]
    for r0 in range(geom.n_frame_rows, geom.L, 256):
        rows += [r0, min(geom.L, r0 + 256) - 1]
    rng = np.random.default_rng(seed)
    rows += rng.choice(w.L, n_random, replace=False).tolist()
    return np.unique(np.asarray(rows, dtype=np.int64))


def test_h3_full_sampled_parity(gpu_lib):
    """The 56-head H3 shape: every head, on rows at every group's item edges and every
    global tile (the oracle's per-row form)."""
    w = WORKLOADS["h3_full"]
    _say(f"h3_full: generating inputs L={w.L} H={w.H}")
    q, k, v = make_inputs(w, seed=0)
    _say("h3_full: running")
    out = _run(gpu_lib, w, q.cuda(), k.cuda(), v.cuda()).cpu()
    rows = _h3_rows(w, 16, seed=2)
    _say(f"h3_full: oracle on {len(rows)} rows x {w.H} heads")
    ref = by_heads(window_attention_rows, q, k, v, Geometry(*w.geometry), rows, [0])
    rel, mx = _errors(out[rows].float(), ref)
    _say(f"h3_full sampled: rel_l2={rel:.3e} max_abs={mx:.3e}")
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
    ((9, 100, 30, 3, 1), 2, 128, torch.float32),   # fp32 out of the split 44-row and 30-row items
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


def _persistent(plan, H):
    """Whether wa_forward takes the persistent work-queue launch for this plan: it does
    when the plan has more than two (head, item) units per compute unit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return plan.info["n_items"] * H > 2 * cus


@pytest.mark.parametrize("name", ["tiny", "small", "dense", "ragged", "h3", "h3_full"])
def test_cover_determinism_locality(gpu_lib, name):
    """Every output element written (NaN prefill), bitwise repeatable over three calls in a
    row (on the persistent launch these reuse the work-queue counters the previous call
    reset), and keys outside a row's window never read: perturbing the frame rows after
    chunk 0's window leaves chunk 0's rows bit-identical, and perturbing the rows before the
    last chunk's window leaves the last chunk's rows bit-identical."""
    w = WORKLOADS[name]
    geom = Geometry(*w.geometry)
    _say(f"cover / determinism / locality on {name}")
    q, k, v = (x.cuda() for x in make_inputs(w, seed=4))
    plan = gpu_lib.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    if name in ("ragged", "h3", "h3_full"):
        assert _persistent(plan, w.H), "expected the persistent work-queue launch"
    outs = []
    for _ in range(3):
        o = torch.full_like(q, float("nan"))
        gpu_lib.wa_forward(plan, q, k, v, out=o)
        outs.append(o)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref = outs[0]
    del outs
    n_frame, C = geom.n_frame_rows, geom.n_chunks
    _, first_end = chunk_span_rows(geom, 0, 0)
    _, span_end = chunk_span_rows(geom, *window_bounds(geom, 0))
    last_begin, _ = chunk_span_rows(geom, C - 1, C - 1)
    span_begin, _ = chunk_span_rows(geom, *window_bounds(geom, (C - 1) * geom.K))
    if span_end == n_frame:
        assert name in ("tiny", "dense") or w.radius >= C - 1
    else:
        k2, v2 = k.clone(), v.clone()
        k2[span_end:n_frame] = 7.0
        v2[span_end:n_frame] = -7.0
        out3 = gpu_lib.wa_forward(plan, q, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(out3[:first_end], ref[:first_end])
        assert not torch.equal(out3[first_end:n_frame], ref[first_end:n_frame])
        del k2, v2, out3
    if span_begin > 0:
        k2, v2 = k.clone(), v.clone()
        k2[:span_begin] = -6.0
        v2[:span_begin] = 5.0
        out3 = gpu_lib.wa_forward(plan, q, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(out3[last_begin:n_frame], ref[last_begin:n_frame])
        assert not torch.equal(out3[:last_begin], ref[:last_begin])


def test_shared_plan_on_two_streams(gpu_lib):
    """Two handles of one geometry (one cached plan, one set of queue counters and
    workspace) used on two streams with no synchronisation in between: the library orders
    the calls, so both results equal the ones computed one after the other."""
    w = WORKLOADS["ragged"]
    _say("shared plan on two streams (ragged)")
    q, k, v = (x.cuda() for x in make_inputs(w, seed=11))
    q2 = torch.flip(q, dims=[0]).contiguous()
    p1 = gpu_lib.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    p2 = gpu_lib.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    assert _persistent(p1, w.H)
    ref1 = gpu_lib.wa_forward(p1, q, k, v)
    ref2 = gpu_lib.wa_forward(p1, q2, k, v)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        o1 = torch.full_like(q, float("nan"))
        o2 = torch.full_like(q, float("nan"))
        torch.cuda.synchronize()
        gpu_lib.wa_forward(p1, q, k, v, out=o1, stream=s1)
        gpu_lib.wa_forward(p2, q2, k, v, out=o2, stream=s2)
        gpu_lib.wa_forward(p2, q, k, v, out=o1, stream=s1)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert torch.equal(o1, ref1)
        assert torch.equal(o2, ref2)


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
    out = torch.full((L, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda(), out=out)
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


def test_score_jump_short_items(gpu_lib):
    """Items of at most 64 rows (here a 44-row window item and a 30-row global item) run
    split over the four waves by key half.  Hot keys in either half of a tile, in a ragged
    tile at a segment end and among the ragged global keys send those tiles to the slow
    path of one half; the halves' merge must keep every row one-hot on its key."""
    # three 300-row groups (chunk spans 0-1, 0-2, 1-2): items of 256 + 44 rows
    T, S, G, K, r, H, d = 9, 100, 30, 3, 1, 2, 128
    _say(f"score jump, short items T={T} S={S} G={G} K={K} r={r} H={H} d={d}")
    L = T * S + G
    q, k, v = make_custom_inputs(L, H, d, torch.bfloat16, seed=11)
    hot = ((260, 100),        # group 0's 44-row item: key 36 of tile 1 (second key half)
           (290, 590),        # key 14 of tile 9, where the chunk keys end after 24 keys
           (299, 920),        # global key: key 20 of the 30-key global tile
           (870, 850),        # group 2's 44-row item (keys from 300): key 38 of tile 8
           (T * S + 5, 300))  # 30-row global item
    for row, key in hot:
        _hot_key(q, k, row, key, 10.0)
    plan = gpu_lib.wa_plan_create(T, S, G, K, r, H, d)
    out = torch.full((L, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda(), out=out)
    torch.cuda.synchronize()
    ref = window_attention_reference(q, k, v, Geometry(T, S, G, K, r))
    got = out.float().cpu()
    rel, mx = _errors(got, ref)
    _say(f"rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert not torch.isnan(got).any()
    assert rel <= REL_L2 and mx <= MAX_ABS
    for row, key in hot:
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


def test_audio_causal_full_parity(gpu_lib):
    """The audio_causal workload (persistent launch) in full against the fp64 causal oracle."""
    w = WORKLOADS["audio_causal"]
    _say(f"audio_causal: L={w.L} H={w.H} d={w.d} fp32")
    q, k, v = make_inputs(w, seed=0)
    plan = gpu_lib.wa_causal_plan_create(w.L, w.H, w.d)
    out = torch.full((w.L, w.H, w.d), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.wa_forward(plan, q.cuda(), k.cuda(), v.cuda(), out=out)
    torch.cuda.synchronize()
    out = out.cpu()
    assert not torch.isnan(out).any()
    _say(f"audio_causal: oracle on all rows x {w.H} heads ({by_heads_workers()} threads)")
    ref = by_heads(causal_attention_reference, q, k, v)
    rel, mx = _errors(out, ref)
    _say(f"audio_causal: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


@pytest.mark.parametrize("case", ["n700", "audio_causal"])
def test_causal_cover_determinism_and_no_future_keys(gpu_lib, case):
    """NaN prefill is fully overwritten, results repeat bit for bit over three calls, and
    perturbing rows >= j of k and v leaves output rows < j bit-identical (future keys are
    never used).  audio_causal takes the persistent work-queue launch."""
    if case == "n700":
        n, H, d, dtype, js = 700, 2, 64, torch.bfloat16, (1, 100, 256, 321, 699)
        q, k, v = (x.cuda() for x in make_custom_inputs(n, H, d, dtype, seed=8))
    else:
        w = WORKLOADS["audio_causal"]
        n, H, d, js = w.L, w.H, w.d, (1, 255, 4096, 10001, w.L - 1)
        q, k, v = (x.cuda() for x in make_inputs(w, seed=8))
    _say(f"causal cover / determinism / future keys: {case}")
    plan = gpu_lib.wa_causal_plan_create(n, H, d)
    if case == "audio_causal":
        assert _persistent(plan, H)
    outs = []
    for _ in range(3):
        o = torch.full_like(q, float("nan"))
        gpu_lib.wa_forward(plan, q, k, v, out=o)
        outs.append(o)
    torch.cuda.synchronize()
    out1 = outs[0]
    assert not torch.isnan(out1).any() and torch.equal(out1, outs[1]) and torch.equal(out1, outs[2])
    for j in js:
        k2, v2 = k.clone(), v.clone()
        k2[j:] = 3.0
        v2[j:] = -5.0
        out3 = gpu_lib.wa_forward(plan, q, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(out3[:j], out1[:j]), j
        assert not torch.equal(out3[j:], out1[j:]), j
