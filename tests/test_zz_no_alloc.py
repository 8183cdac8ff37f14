"""wa_forward_noalloc (the entry point that allocates nothing) against wa_forward.

Both run the same kernels on the same plan, so their outputs must agree bit for bit; the
no-allocation call is checked on calls in a row with a smaller input second (the static
workspace keeps the previous call's contents, so the queue counters and partials must be
re-established by each call), on fp32 inputs (bf16 staging in the workspace), on a plan it
must reject (56 heads at the H3 scale: its partials exceed the workspace), and for not
allocating: a first call with a plan that wa_forward never ran leaves free device memory
unchanged.
"""

import sys

import pytest
import torch

from chunk_windowed_softmax_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _plan(wa, w, H=None):
    return wa.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, H or w.H, w.d)


def _both(wa, w, seed):
    q, k, v = (x.cuda() for x in make_inputs(w, seed=seed))
    plan = _plan(wa, w)
    ref = wa.wa_forward(plan, q, k, v)
    out = torch.full_like(q, float("nan"))
    wa.wa_forward_noalloc(plan, q, k, v, out)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_matches_wa_forward(gpu_lib):
    # the H3 share (persistent launch, 21 global-leg splits: 78 MB of partials), then the
    # smaller workload, then the H3 share again and the fp32 one
    for name, seed in (("h3", 21), ("small", 22), ("h3", 23), ("tiny", 24)):
        _say(f"{name} seed {seed}")
        out, ref = _both(gpu_lib, WORKLOADS[name], seed)
        assert not torch.isnan(out).any(), name
        assert torch.equal(out, ref), name


def test_noalloc_twice_in_a_row_without_sync(gpu_lib):
    """Two calls in a row on one stream, the second with a smaller input, no
    synchronisation in between; each equals wa_forward's result."""
    big, small = WORKLOADS["ragged"], WORKLOADS["small"]
    qb, kb, vb = (x.cuda() for x in make_inputs(big, seed=31))
    qs, ks, vs = (x.cuda() for x in make_inputs(small, seed=32))
    pb, ps = _plan(gpu_lib, big), _plan(gpu_lib, small)
    ref_b = gpu_lib.wa_forward(pb, qb, kb, vb)
    ref_s = gpu_lib.wa_forward(ps, qs, ks, vs)
    ob, os_ = torch.full_like(qb, float("nan")), torch.full_like(qs, float("nan"))
    torch.cuda.synchronize()
    _say("ragged then small, back to back")
    gpu_lib.wa_forward_noalloc(pb, qb, kb, vb, ob)
    gpu_lib.wa_forward_noalloc(ps, qs, ks, vs, os_)
    torch.cuda.synchronize()
    assert torch.equal(ob, ref_b)
    assert torch.equal(os_, ref_s)


def test_noalloc_rejects_plans_beyond_the_workspace(gpu_lib):
    w = WORKLOADS["h3_full"]
    plan = _plan(gpu_lib, w)
    shape = (w.L, w.H, w.d)
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(gpu_lib.WaError) as e:
        gpu_lib.wa_forward_noalloc(plan, q, q, q, out)
    assert e.value.code == gpu_lib.WA_ERR_UNSUPPORTED and "static" in str(e.value)


def test_noalloc_allocates_no_device_memory(gpu_lib):
    """A plan that wa_forward never ran (so it has no device tables or workspace of its
    own): the no-allocation call leaves free device memory as it was, whereas its first
    wa_forward allocates the plan's 70+ MB of partials."""
    w = WORKLOADS["h3"]
    q, k, v = (x.cuda() for x in make_inputs(w, seed=41))
    out = torch.empty_like(q)
    warm = _plan(gpu_lib, w)  # load the kernels and the workspace address once
    gpu_lib.wa_forward_noalloc(warm, q, k, v, out)
    torch.cuda.synchronize()
    # same tensors, a geometry with one global row less (a new plan; the last row's output
    # is left as it is)
    fresh = gpu_lib.wa_plan_create(w.T, w.S, w.G - 1, w.K, w.radius, w.H, w.d)
    qf, kf, vf, of = (t[: w.L - 1] for t in (q, k, v, out))
    ref = torch.empty_like(qf)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    gpu_lib.wa_forward_noalloc(fresh, qf, kf, vf, of)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    _say(f"free device memory before/after: {free0} / {free1}")
    assert free0 - free1 < 16 << 20
    gpu_lib.wa_forward(fresh, qf, kf, vf, out=ref)
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    _say(f"after the first wa_forward of that plan: {free2}")
    assert free1 - free2 >= 64 << 20
    assert torch.equal(of, ref)
