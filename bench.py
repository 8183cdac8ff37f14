#!/usr/bin/env python3
"""Benchmark of the decomposed chunk-windowed softmax attention on one MI355X.

Metric: kept-pair TFLOP/s (4*d FLOP per kept (query, key) pair, all heads) and ms per
call at the H3-scale one-GPU share (T=102 latent frames x S=960 tokens, K=3, radius 1,
G=1024 global tokens, 7 heads of d=128, bf16), plus the fraction of MI355X's dense bf16
MFMA peak.  One "step" is one wa_forward call (both legs and the merge) over inputs
already resident in HBM.

``--op fp8`` times the FP8 (e4m3) variant, wa_forward_fp8, on the same workload quantised
per tensor, against the fp8 dense MFMA peak.

``--op prologue`` instead times the fused QK-RMSNorm + rotary prologue
(wa_qk_norm_rope) on the same workload's q and k: a memory-bound pass, reported as
algorithmic HBM GB/s against MI355X's 8 TB/s.

Prints ONE JSON line.  ``--gpus N`` with N > 1 is refused: this build runs on one GPU.
"""

from __future__ import annotations

import argparse
import glob
import json
import os
import statistics
import sys
import threading
import time

MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
MFMA_FP8_PEAK_TFLOPS = 5033.2   # twice the bf16 rate
HBM_PEAK_GBS = 8000.0


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="h3",
                    help="workload name (h3, h3_full, small, ragged, dense, audio_causal, audio_causal_small)")
    ap.add_argument("--op", default="attention", choices=["attention", "prologue", "fp8", "blocksparse"],
                    help="attention: wa_forward (default); prologue: wa_qk_norm_rope; fp8: wa_forward_fp8; "
                         "blocksparse: the block-sparse plan against the decomposed one")
    ap.add_argument("--block", default="256x128", help="query x key block sizes for --op blocksparse")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of the workload the CPU oracle runs (0: all, at most 16)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows the CPU oracle runs for --op prologue (0: all)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a plain device copy of q (known bytes) to calibrate HBM byte counters")
    return ap.parse_args()


def _pool_size() -> int:
    """Worker threads for the CPU oracle: the cores this process may use, at most 16 (the
    host share of one GPU on a shared node)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _by_heads(fn, q, k, v, heads: int, *args):
    """Run `fn` (an oracle function over [L, H', d] tensors) on heads 0..heads-1, one head per
    task, in a pool of worker threads with one BLAS thread each (numpy releases the
    interpreter lock inside its products and exponentials).  Returns (seconds, threads)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    threads = min(_pool_size(), heads)
    with threadpool_limits(1):
        with ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            list(ex.map(lambda h: fn(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], *args), range(heads)))
            dt = time.perf_counter() - t0
    return dt, threads


def cpu_baseline(w, q, k, v, heads: int) -> dict:
    """Time the fp64 oracle (as it stands) on the first `heads` heads of the workload, all
    rows, one head per task in a pool of worker threads."""
    from oracle import (Geometry, causal_attention_reference, causal_pairs_per_head, kept_pairs_per_head,
                        window_attention_reference)

    heads = max(1, min(heads, w.H))
    if w.causal:
        dt, threads = _by_heads(causal_attention_reference, q, k, v, heads)
        pairs = causal_pairs_per_head(w.L)
    else:
        geom = Geometry(*w.geometry)
        dt, threads = _by_heads(window_attention_reference, q, k, v, heads, geom)
        pairs = kept_pairs_per_head(geom)
    flop = pairs * heads * 4 * w.d
    return {
        "value": round(flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"fp64 numpy {'causal' if w.causal else 'per-frame'} oracle on {heads} of {w.H} heads of the "
                  f"{w.name} workload (all {w.L} rows), one head per worker thread, {threads} threads with one "
                  f"BLAS thread each, {dt:.1f} s wall",
        "seconds": round(dt, 3),
    }


def recorded_traffic(workload: str, kernel: str = "attn_kernel"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counters
    (profiles/<kernel>_<workload>.json), or None when absent or taken on other source."""
    from chunk_windowed_softmax_amd.rocprof_summary import kernel_source_sha256

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_sha256(kernel):
        return None, rec
    return rec["traffic_bytes"], rec


class SclkSampler:
    """The GPU's current shader clock while the timed calls run: the "S:" (current) line of
    the card's pp_dpm_sclk in sysfs, which is the figure `rocm-smi --showclocks` prints, read
    every 5 ms by a thread.  The card is the one at the PCI address of torch's device 0 (else
    the only AMD card with that file).  `stats()` is None where the file is missing."""

    def __init__(self):
        self.path = self._find()
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    @staticmethod
    def _find():
        cards = []
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            try:
                with open(os.path.join(dev, "vendor")) as f:
                    if f.read().strip() == "0x1002" and os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                        cards.append(dev)
            except OSError:
                pass
        try:
            import torch

            pr = torch.cuda.get_device_properties(0)
            addr = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}."
            for dev in cards:
                if os.path.basename(os.path.realpath(dev)).startswith(addr):
                    return os.path.join(dev, "pp_dpm_sclk")
        except (AttributeError, RuntimeError):
            pass
        return os.path.join(cards[0], "pp_dpm_sclk") if len(cards) == 1 else None

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz = self._read()
            except (OSError, ValueError, IndexError):
                return
            if mhz is not None:
                self.samples.append(mhz)
            self._stop.wait(0.005)

    def start(self):
        if self.path is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=1.0)

    def stats(self):
        if not self.samples:
            return None
        return {"median": statistics.median(self.samples), "min": min(self.samples), "max": max(self.samples),
                "samples": len(self.samples),
                "source": f"current shader clock, {self.path} (as rocm-smi --showclocks), every 5 ms over the "
                          "timed calls"}


def _time_calls(fn, steps: int, warmup: int, stream, sampler: SclkSampler | None = None):
    """Warm up, then time `steps` calls back to back: HIP events on the launch stream at the
    start and the end of the timed region (no event between calls, so the host enqueues ahead
    of the device) and the wall clock around it (synchronised on both sides).  Returns
    (device ms per call, wall ms per call).  A sampler, if given, runs over the timed region."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if sampler is not None:
        sampler.start()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if sampler is not None:
        sampler.stop()
    return start.elapsed_time(end) / steps, wall * 1e3 / steps


def _time_each(fn, steps: int, stream):
    """A second pass of `steps` calls with a HIP event on the launch stream between
    consecutive calls: (median, min) device ms per call."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ts = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return statistics.median(ts), min(ts)


def _calibration_copy(x):
    import torch

    scratch = torch.empty_like(x)
    for _ in range(3):
        scratch.copy_(x)
    torch.cuda.synchronize()
    print(f"calibration copy: {x.numel() * x.element_size()} bytes read and written per copy", flush=True)


def prologue_bytes(L: int, H: int, d: int, elem: int, weights: bool) -> int:
    """Algorithmic HBM bytes of one QK-norm + rotary call: q and k read and written once,
    the fp32 cos and sin tables [L, d/2] read once, the two fp32 weight vectors."""
    return 4 * L * H * d * elem + 2 * L * (d // 2) * 4 + (2 * d * 4 if weights else 0)


def bench_fp8(args, w) -> int:
    import torch

    import chunk_windowed_softmax_amd as wa
    from chunk_windowed_softmax_amd.workloads import make_fp8_inputs

    dev = torch.device("cuda:0")
    q8c, k8c, v8c, sq, sk, sv = make_fp8_inputs(w, seed=0)
    q8, k8, v8 = (x.to(dev) for x in (q8c, k8c, v8c))
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    t0 = time.perf_counter()
    plan = wa.wa_causal_plan_create(w.L, w.H, w.d) if w.causal else wa.wa_plan_create(
        w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info
    flop = info["kept_pairs_per_head"] * w.H * 4 * w.d
    stream = torch.cuda.current_stream(dev)
    if args.calibration_copy:
        _calibration_copy(q8)
    call = lambda: wa.wa_forward_fp8(plan, q8, k8, v8, sq, sk, sv, out=out, stream=stream)  # noqa: E731
    sclk = SclkSampler()
    dev_ms, ms_step = _time_calls(call, args.steps, args.warmup, stream, sclk)
    med_ms, min_ms = _time_each(call, args.steps, stream)
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (dev_ms * 1e-3) / 1e12
    traffic, traffic_rec = recorded_traffic(w.name, "attn_fp8_kernel")
    res = {
        "metric": ("kept-pair TFLOP/s of the FP8 (e4m3) window call at the H3-scale share on 1 MI355X"
                   if w.name.startswith("h3") else f"kept-pair TFLOP/s of the FP8 (e4m3) {w.name} call on 1 MI355X"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"fp8 {w.name}", "T": w.T, "S": w.S, "G": w.G, "K": w.K, "radius": w.radius,
            "H": w.H, "d": w.d, "L": w.L, "kept_pairs": info["kept_pairs_per_head"] * w.H,
            "flop_per_call": flop, "scales": "per tensor", "parallelism": "single GPU",
        },
        "ms_per_call": {"device_mean": round(dev_ms, 4), "median": round(med_ms, 4), "min": round(min_ms, 4),
                        "median_min_from": "a second pass of as many calls, HIP events between consecutive calls"},
        "tflops_at_median": round(flop / (med_ms * 1e-3) / 1e12, 2),
        "sclk_mhz": sclk.stats(),
        "plan_create_ms": round(plan_ms, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fp8_kernel, then its merge kernel when the global leg is split: one wa_forward_fp8 call",
            "duration": "device time of the timed region (HIP events on the launch stream before the first and "
                        "after the last call) / calls: both kernels",
            "achieved": round(achieved, 2),
            "peak": MFMA_FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4),
            "traffic": None if traffic is None else int(traffic),
            "algorithmic_bytes": int(3 * w.L * w.H * w.d + 2 * w.L * w.H * w.d + 2 * info["workspace_bytes"]),
            "traffic_source": None if traffic_rec is None else
            f"profiles/attn_fp8_kernel_{w.name}.md" + ("" if traffic is not None else " (stale: kernel changed)"),
        },
    }
    if not args.no_cpu_baseline:
        from oracle import decode_e4m3

        vals = [torch.from_numpy(decode_e4m3(c) * s) for c, s in ((q8c, sq), (k8c, sk), (v8c, sv))]
        res["cpu_baseline"] = cpu_baseline(w, *vals, args.cpu_heads or min(16, w.H))
        res["cpu_baseline"]["sample"] += " (decoded fp8 inputs)"
    print(json.dumps(res), flush=True)
    return 0


def bench_prologue(args, w) -> int:
    import torch

    import chunk_windowed_softmax_amd as wa
    from chunk_windowed_softmax_amd.workloads import make_norm_weights, make_prologue_inputs, make_rope_tables

    dev = torch.device("cuda:0")
    q_cpu, k_cpu = make_prologue_inputs(w.L, w.H, w.d, w.dtype, seed=0)
    cos_cpu, sin_cpu = make_rope_tables(w.L, w.d)
    wq_cpu, wk_cpu = make_norm_weights(w.d, 0)
    q, k, cos, sin, wq, wk = (x.to(dev) for x in (q_cpu, k_cpu, cos_cpu, sin_cpu, wq_cpu, wk_cpu))
    q_out, k_out = torch.empty_like(q), torch.empty_like(k)
    stream = torch.cuda.current_stream(dev)
    if args.calibration_copy:
        _calibration_copy(q)

    def call():
        wa.wa_qk_norm_rope(q, k, cos, sin, wq, wk, q_out=q_out, k_out=k_out, stream=stream)

    dev_ms, ms_step = _time_calls(call, args.steps, args.warmup, stream)
    elem = q.element_size()
    nbytes = prologue_bytes(w.L, w.H, w.d, elem, True)
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (dev_ms * 1e-3) / 1e9
    traffic, traffic_rec = recorded_traffic(w.name, "qk_norm_rope_kernel")
    res = {
        "metric": "QK-RMSNorm + rotary prologue algorithmic HBM GB/s at the H3-scale window call on 1 MI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"qk_norm_rope on {w.name} q/k", "L": w.L, "H": w.H, "d": w.d, "weights": True,
            "pairs": "rotate-half", "bytes_per_call": nbytes, "parallelism": "single GPU",
        },
        "ms_per_call": {"device_mean": round(dev_ms, 5)},
        "roofline": {
            "bound": "hbm",
            "kernel": "qk_norm_rope_kernel: one wa_qk_norm_rope call",
            "duration": "device time of the timed region (HIP events on the launch stream before the first and "
                        "after the last call) / calls",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic),
            "algorithmic_bytes": int(nbytes),
            "traffic_source": None if traffic_rec is None else
            f"profiles/qk_norm_rope_kernel_{w.name}.md" + ("" if traffic is not None else " (stale: kernel changed)"),
        },
    }
    if not args.no_cpu_baseline:
        from oracle import qk_norm_rope_reference

        n = min(args.cpu_rows, w.L) if args.cpu_rows > 0 else w.L
        t0 = time.perf_counter()
        qk_norm_rope_reference(q_cpu[:n], k_cpu[:n], cos_cpu[:n], sin_cpu[:n], wq_cpu, wk_cpu)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {
            "value": round(prologue_bytes(n, w.H, w.d, elem, True) / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "host_cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle on the first {n} of {w.L} rows (all {w.H} heads, q and k), one thread "
                      f"with one BLAS thread, {dt:.2f} s wall",
            "seconds": round(dt, 3),
        }
    print(json.dumps(res), flush=True)
    return 0


def bench_blocksparse(args, w) -> int:
    """The block-sparse plan (FlexAttention-style block mask, [VDN] §二) and the decomposed
    plan on the same inputs, timed in alternating rounds in one process; the line reports the
    block-sparse call and the A/B."""
    import torch

    import chunk_windowed_softmax_amd as wa
    from chunk_windowed_softmax_amd.workloads import make_inputs

    bq, bk = (int(x) for x in args.block.lower().split("x"))
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in make_inputs(w, seed=0))
    out = torch.empty_like(q)
    t0 = time.perf_counter()
    plan_b = wa.wa_blocksparse_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d, bq, bk)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan_d = wa.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    info_b, info_d = plan_b.info, plan_d.info
    flop = info_b["kept_pairs_per_head"] * w.H * 4 * w.d
    stream = torch.cuda.current_stream(dev)
    rounds = 4
    call_b = wa.prepared_forward(plan_b, q, k, v, out, stream)
    call_d = wa.prepared_forward(plan_d, q, k, v, out, stream)
    dev_b, dev_d, walls = [], [], []
    for r in range(rounds):
        d, ms = _time_calls(call_b, max(1, args.steps // rounds), args.warmup if r == 0 else 2, stream)
        dev_b.append(d)
        walls.append(ms)
        d, _ = _time_calls(call_d, max(1, args.steps // rounds), args.warmup if r == 0 else 2, stream)
        dev_d.append(d)
    steps = rounds * max(1, args.steps // rounds)
    ms_step = statistics.fmean(walls)
    mean_b, mean_d = statistics.fmean(dev_b), statistics.fmean(dev_d)
    achieved = flop / (mean_b * 1e-3) / 1e12
    res = {
        "metric": f"kept-pair TFLOP/s of the block-sparse ({bq},{bk}) {w.name} call on 1 MI355X",
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"blocksparse {bq}x{bk} {w.name}", "T": w.T, "S": w.S, "G": w.G, "K": w.K,
            "radius": w.radius, "H": w.H, "d": w.d, "L": w.L, "block_q": bq, "block_kv": bk,
            "kept_pairs": info_b["kept_pairs_per_head"] * w.H, "flop_per_call": flop,
            "parallelism": "single GPU",
        },
        "ms_per_call": {"device_mean": round(mean_b, 4), "device_min_round": round(min(dev_b), 4)},
        "plan_create_ms": round(plan_ms, 3),
        "ab": {
            "decomposed_ms_mean": round(mean_d, 4),
            "blocksparse_ms_mean": round(mean_b, 4),
            "blocksparse_time_over_decomposed": round(mean_b / mean_d, 4),
            "computed_pairs_blocksparse": info_b["computed_pairs_per_head"] * w.H,
            "computed_pairs_decomposed": info_d["computed_pairs_per_head"] * w.H,
            "rounds": rounds,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_kernel (tile-list instantiation), then combine_kernel: one wa_forward call",
            "duration": "device time of the timed block-sparse regions (HIP events on the launch stream before "
                        "the first and after the last call of each round) / calls: both kernels",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_bytes": int(4 * w.L * w.H * w.d * q.element_size() + 2 * info_b["workspace_bytes"]),
        },
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported by this build "
              f"(the path shards by heads across GPUs, which is not built here).", file=sys.stderr)
        return 2

    import torch

    import chunk_windowed_softmax_amd as wa
    from chunk_windowed_softmax_amd.workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wa.load_library()
    w = WORKLOADS[args.workload]
    if args.op == "prologue":
        return bench_prologue(args, w)
    if args.op == "fp8":
        return bench_fp8(args, w)
    if args.op == "blocksparse":
        return bench_blocksparse(args, w)
    q_cpu, k_cpu, v_cpu = make_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (q_cpu, k_cpu, v_cpu))
    out = torch.empty_like(q)

    t0 = time.perf_counter()
    if w.causal:
        plan = wa.wa_causal_plan_create(w.L, w.H, w.d)
    else:
        plan = wa.wa_plan_create(w.T, w.S, w.G, w.K, w.radius, w.H, w.d)
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info
    flop = info["kept_pairs_per_head"] * w.H * 4 * w.d

    stream = torch.cuda.current_stream(dev)
    if args.calibration_copy:
        # one read + one write of q.numel()*2 bytes per copy; profiled beside the attention
        _calibration_copy(q)

    call = wa.prepared_forward(plan, q, k, v, out, stream)
    sclk = SclkSampler()
    dev_ms, ms_step = _time_calls(call, args.steps, args.warmup, stream, sclk)
    med_ms, min_ms = _time_each(call, args.steps, stream)

    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (dev_ms * 1e-3) / 1e12
    # Algorithmic HBM bytes: q, k, v read once and out written once, plus the global leg's
    # fp32 partials (written once, read once by the merge).
    elem = 2 if w.dtype == torch.bfloat16 else 4
    algo_bytes = 4 * w.L * w.H * w.d * elem + 2 * info["workspace_bytes"]
    traffic, traffic_rec = recorded_traffic(w.name)
    res = {
        "metric": ("kept-pair TFLOP/s at the H3-scale window call on 1 MI355X" if w.name.startswith("h3")
                   else f"kept-pair TFLOP/s of the {w.name} attention call on 1 MI355X"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "T": w.T, "S": w.S, "G": w.G, "K": w.K, "radius": w.radius,
            "H": w.H, "d": w.d, "L": w.L, "kept_pairs": info["kept_pairs_per_head"] * w.H,
            "flop_per_call": flop, "n_groups": info["n_groups"], "n_splits": info["n_splits"],
            "parallelism": "single GPU",
        },
        "ms_per_call": {"device_mean": round(dev_ms, 4), "median": round(med_ms, 4), "min": round(min_ms, 4),
                        "median_min_from": "a second pass of as many calls, HIP events between consecutive calls"},
        "tflops_at_median": round(flop / (med_ms * 1e-3) / 1e12, 2),
        "pct_of_bf16_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "sclk_mhz": sclk.stats(),
        "plan_create_ms": round(plan_ms, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_kernel, then combine_kernel when the global leg is split: one wa_forward call",
            "duration": "device time of the timed region (HIP events on the launch stream before the first and "
                        "after the last call) / calls: both kernels",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None if traffic is None else int(traffic),
            "algorithmic_bytes": int(algo_bytes),
            "traffic_source": None if traffic_rec is None else
            f"profiles/attn_kernel_{w.name}.md" + ("" if traffic is not None else " (stale: kernel changed)"),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, args.cpu_heads or min(16, w.H))
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
