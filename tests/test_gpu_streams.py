"""Every entry point enqueues on the stream it is given: results computed on a side stream
(inputs produced there, nothing synchronised in between) equal those of the current stream
bit for bit."""

import pytest
import torch

from chunk_windowed_softmax_amd.workloads import (WORKLOADS, make_fp8_inputs, make_inputs, make_norm_weights,
                                                  make_prologue_inputs, make_rope_tables)

pytestmark = pytest.mark.gpu


def test_forward_on_a_side_stream(gpu_lib):
    w = WORKLOADS["small"]
    q, k, v = (x.cuda() for x in make_inputs(w, seed=8))
    plan = gpu_lib.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    ref = gpu_lib.wa_forward(plan, q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q2 = q * 1  # produced on the side stream
        out = gpu_lib.wa_forward(plan, q2, k, v, stream=side)
    side.synchronize()
    assert torch.equal(out, ref)


def test_fp8_and_prologue_on_a_side_stream(gpu_lib):
    w = WORKLOADS["small"]
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(w, seed=9)
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    plan = gpu_lib.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    ref8 = gpu_lib.wa_forward_fp8(plan, q8, k8, v8, sq, sk, sv)
    qp, kp = (x.cuda() for x in make_prologue_inputs(500, 3, 128, torch.bfloat16, seed=9))
    cos, sin = (x.cuda() for x in make_rope_tables(500, 128))
    wq, wk = (x.cuda() for x in make_norm_weights(128, 9))
    refq, refk = gpu_lib.wa_qk_norm_rope(qp, kp, cos, sin, wq, wk)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        v8b = v8.clone()
        out8 = gpu_lib.wa_forward_fp8(plan, q8, k8, v8b, sq, sk, sv, stream=side)
        qpb = qp.clone()
        oq, ok = gpu_lib.wa_qk_norm_rope(qpb, kp, cos, sin, wq, wk, stream=side)
    side.synchronize()
    assert torch.equal(out8, ref8)
    assert torch.equal(oq, refq) and torch.equal(ok, refk)
