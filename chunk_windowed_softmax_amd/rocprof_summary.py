"""Summarise rocprofv3 output of ``bench.py`` runs into ``profiles/``.

Inputs (all CSV, written with ``rocprofv3 --output-format csv``):

* a ``--kernel-trace --stats`` run: per-kernel call counts and durations;
* a ``--pmc FETCH_SIZE`` run and a ``--pmc WRITE_SIZE`` run of ``bench.py --calibration-copy``:
  both counters (KiB per dispatch) are read for the profiled kernel (``--kernel``: the
  attention kernel by default, or the QK-norm + rotary prologue) and for the plain
  device copy of a known byte count that the calibration step runs first.  Each counter is
  scaled by (known copy bytes / counter reading of the copy), so the kernel's
  HBM bytes are expressed in the units of a transfer whose size is known.

Output: ``<out>.md`` (human summary with the commands) and ``<out>.json`` (figures that
``bench.py`` reports as ``roofline.traffic`` while the kernel source is unchanged).

Usage::

    python -m chunk_windowed_softmax_amd.rocprof_summary --trace DIR --fetch DIR --write DIR \
        --copy-bytes N --out profiles/attn_kernel_h3_share --command-trace "..." \
        --command-fetch "..." --command-write "..."
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
ATTN = "attn_kernel"
COMBINE = "combine_kernel"
PROLOGUE = "qk_norm_rope_kernel"
FP8 = "attn_fp8_kernel"
COPY = "copyBuffer"
SOURCES = {ATTN: "kernels.hip", PROLOGUE: "prologue.hip", FP8: "attn_fp8.hip"}


def _code_only(text: str) -> str:
    """The source without its comments and with runs of whitespace collapsed, so that
    counters stay tied to the code they were taken on across comment edits.  (The kernel
    sources hold no string or character literal with a comment marker in it.)"""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha256(kernel: str = ATTN) -> str:
    """sha256 of the kernel's source file, comments and whitespace runs removed."""
    with open(os.path.join(PKG, "csrc", SOURCES[kernel]), encoding="utf-8") as f:
        return hashlib.sha256(_code_only(f.read()).encode()).hexdigest()


def _rows(pattern: str) -> List[Dict[str, str]]:
    out: List[Dict[str, str]] = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def _short(name: str) -> str:
    for key in (ATTN, COMBINE, PROLOGUE, FP8, COPY):
        if key in name:
            return key
    return name[:60]


def trace_durations(trace_dir: str, skip: int = 0) -> Dict[str, List[float]]:
    """Dispatch durations (ns) per kernel in launch order, without the first `skip`
    dispatches of each kernel (the untimed warm-up calls of a bench run)."""
    rows = _rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    rows.sort(key=lambda r: float(r["Start_Timestamp"]))
    d: Dict[str, List[float]] = {}
    for r in rows:
        d.setdefault(_short(r["Kernel_Name"]), []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return {k: v[skip:] if len(v) > skip else v for k, v in d.items()}


def counter_means(pmc_dir: str, counter: str) -> Dict[str, float]:
    """Mean counter value per kernel.  For the copy kernel only the largest dispatches (the
    calibration copy) count; smaller copies (plan upload) are ignored."""
    rows = _rows(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    vals: Dict[str, List[float]] = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    if COPY in vals:
        top = max(vals[COPY])
        vals[COPY] = [x for x in vals[COPY] if x >= 0.5 * top]
    return {k: statistics.fmean(v) for k, v in vals.items()}


def sq_means(pmc_dir: str) -> Dict[str, Dict[str, float]]:
    """Mean of every counter per kernel, with the mean dispatch duration in ns."""
    rows = _rows(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    vals: Dict[str, Dict[str, List[float]]] = {}
    for r in rows:
        d = vals.setdefault(_short(r["Kernel_Name"]), {})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        d.setdefault("_duration_ns", []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return {k: {c: statistics.fmean(v) for c, v in d.items()} for k, d in vals.items()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--workload", default="h3")
    ap.add_argument("--kernel", default=ATTN, choices=sorted(SOURCES))
    ap.add_argument("--flop-per-call", type=float, default=0.0)
    ap.add_argument("--algorithmic-bytes", type=float, required=True)
    ap.add_argument("--command-trace", default="")
    ap.add_argument("--command-fetch", default="")
    ap.add_argument("--command-write", default="")
    ap.add_argument("--sq", default="", help="pmc run with SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_*, GRBM_GUI_ACTIVE")
    ap.add_argument("--command-sq", default="")
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--simds", type=int, default=1024)
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--skip", type=int, default=0,
                    help="dispatches of each kernel to drop from the trace statistics (the warm-up calls)")
    ap.add_argument("--per-call", default="",
                    help="comma-separated kernels that one call launches, summed per call (e.g. attn_kernel,combine_kernel)")
    a = ap.parse_args()
    kern = a.kernel  # the profiled kernel

    dur = trace_durations(a.trace, a.skip)
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    copy_kib = a.copy_bytes / 1024.0
    f_fetch = copy_kib / fetch[COPY]
    f_write = copy_kib / write[COPY]
    attn_fetch = fetch[kern] * f_fetch * 1024.0
    attn_write = write[kern] * f_write * 1024.0
    attn_ns = statistics.fmean(dur[kern])
    res = {
        "workload": a.workload,
        "kernel": kern,
        "kernel_source_sha256": kernel_source_sha256(kern),
        "avg_duration_ms": attn_ns / 1e6,
        "median_duration_ms": statistics.median(dur[kern]) / 1e6,
        "calls": len(dur[kern]),
        "tflops_at_avg_duration": a.flop_per_call / (attn_ns * 1e-9) / 1e12 if a.flop_per_call else None,
        "fetch_kib_raw": fetch[kern],
        "write_kib_raw": write[kern],
        "copy_scale_fetch": f_fetch,
        "copy_scale_write": f_write,
        "fetch_bytes": attn_fetch,
        "write_bytes": attn_write,
        "traffic_bytes": attn_fetch + attn_write,
        "algorithmic_bytes": a.algorithmic_bytes,
        "hbm_gbs_at_avg_duration": (attn_fetch + attn_write) / (attn_ns * 1e-9) / 1e9,
        "algorithmic_gbs_at_avg_duration": a.algorithmic_bytes / (attn_ns * 1e-9) / 1e9,
        "skipped_dispatches_per_kernel": a.skip,
    }
    call_kernels = [x for x in a.per_call.split(",") if x]
    if call_kernels:
        call_ns = sum(statistics.fmean(dur[x]) for x in call_kernels if x in dur)
        res["per_call_kernels"] = call_kernels
        res["per_call_avg_ms"] = call_ns / 1e6
        if a.flop_per_call:
            res["tflops_at_per_call_avg"] = a.flop_per_call / (call_ns * 1e-9) / 1e12
    sq_lines = []
    if a.sq:
        sq = sq_means(a.sq)[kern]
        xcd_cycles = sq["GRBM_GUI_ACTIVE"] / a.xcds  # GPU cycles of one XCD over the dispatch
        clock_ghz = xcd_cycles / sq["_duration_ns"]
        mfma_busy = sq["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * a.simds)
        lds_conf = sq["SQ_LDS_BANK_CONFLICT"] / max(1.0, sq["SQ_LDS_IDX_ACTIVE"])
        lds_active = sq["SQ_LDS_IDX_ACTIVE"] / (xcd_cycles * a.cus)
        res.update({"effective_clock_ghz": clock_ghz, "mfma_busy_frac": mfma_busy,
                    "lds_bank_conflict_frac": lds_conf, "lds_active_frac": lds_active})
        sq_lines = [
            f"SQ / GRBM counters (`{a.command_sq}`), mean over dispatches:",
            "",
            "| counter | value |",
            "|---|---|",
        ] + [f"| {c} | {v:.6g} |" for c, v in sorted(sq.items()) if not c.startswith("_")] + [
            "",
            f"- effective clock: GRBM_GUI_ACTIVE / {a.xcds} XCDs / duration = {clock_ghz:.2f} GHz",
            f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (XCD cycles x {a.simds} SIMDs) = {100 * mfma_busy:.1f}%",
            f"- LDS active: SQ_LDS_IDX_ACTIVE / (XCD cycles x {a.cus} CUs) = {100 * lds_active:.1f}%",
            f"- LDS bank conflicts: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = {100 * lds_conf:.2f}%",
            "",
        ]
    with open(a.out + ".json", "w") as f:
        json.dump(res, f, indent=1)
    lines = [
        f"# rocprofv3 summary: `{kern}` on the {a.workload} workload",
        "",
        "Commands (run from the repository root on one MI355X):",
        "",
        f"- kernel trace: `{a.command_trace}`",
        f"- FETCH_SIZE:   `{a.command_fetch}`",
        f"- WRITE_SIZE:   `{a.command_write}`",
        "",
        (f"Statistics over the timed calls: the first {a.skip} dispatches of each kernel (the warm-up "
         "calls) are dropped." if a.skip else "Statistics over all dispatches."),
        "",
        "| kernel | calls | avg ms | median ms | min ms | max ms |",
        "|---|---|---|---|---|---|",
    ]
    for k, v in sorted(dur.items()):
        lines.append(f"| {k} | {len(v)} | {statistics.fmean(v)/1e6:.4f} | {statistics.median(v)/1e6:.4f} | "
                     f"{min(v)/1e6:.4f} | {max(v)/1e6:.4f} |")
    if a.flop_per_call:
        lines += ["", f"Kept-pair FLOP per call: {a.flop_per_call:.6g}; at the average `{kern}` duration: "
                  f"{res['tflops_at_avg_duration']:.1f} TFLOP/s."]
    if call_kernels:
        lines += ["", f"One call ({' + '.join(call_kernels)}): {res['per_call_avg_ms']:.4f} ms on average"
                  + (f", {res['tflops_at_per_call_avg']:.1f} TFLOP/s." if a.flop_per_call else ".")]
    lines += [
        "",
        f"Algorithmic bytes per call: {a.algorithmic_bytes:.6g}; at the average `{kern}` duration: "
        f"{res['algorithmic_gbs_at_avg_duration']:.0f} GB/s.",
        "",
        "HBM counters (KiB per dispatch, mean over dispatches), scaled by a plain copy of "
        f"{a.copy_bytes} bytes:",
        "",
        "| counter | copy raw | scale | kernel raw | kernel bytes |",
        "|---|---|---|---|---|",
        f"| FETCH_SIZE | {fetch[COPY]:.1f} | {f_fetch:.4f} | {fetch[kern]:.1f} | {attn_fetch:.4g} |",
        f"| WRITE_SIZE | {write[COPY]:.1f} | {f_write:.4f} | {write[kern]:.1f} | {attn_write:.4g} |",
        "",
        f"Traffic per launch {res['traffic_bytes']:.4g} B vs algorithmic {a.algorithmic_bytes:.4g} B "
        f"(ratio {res['traffic_bytes'] / a.algorithmic_bytes:.2f}); {res['hbm_gbs_at_avg_duration']:.0f} GB/s.",
        "",
        f"Kernel source sha256 (comments and whitespace runs removed): `{res['kernel_source_sha256']}`",
        "",
    ] + sq_lines
    with open(a.out + ".md", "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
